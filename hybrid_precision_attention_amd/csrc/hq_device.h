// Device-side helpers shared by the gfx950 kernels of libhq.
//
// The K4V4 group rule (per token, per 32 consecutive head_dim elements):
// min m, max M, scale s = fp16_rne((M - m) / 15), code = clamp(rne((x - m)/s),
// 0, 15), all codes 0 when s == 0; two codes per byte, lower element in the
// low nibble.  The decision is taken in fp64: x - m and M - m are exact there
// (fp16 differences need at most 41 significant bits), and the single
// correctly-rounded fp64 division cannot move a quotient across a half-integer
// boundary, so the codes equal the exact-arithmetic definition.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kD = 128;        // head_dim
constexpr int kGroup = 32;     // elements per quantisation group
constexpr int kRowBytes = kD / 2;        // packed code bytes per token
constexpr int kMetaWords = kD / kGroup;  // {scale, min} words per token

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Nearest fp16 (ties to even) of a non-negative double below 65504: exact
// integer rounding of x scaled to the 11-bit significand of its binade
// (subnormals share the binade of 2^-14).
__device__ __forceinline__ uint16_t d2h_rne_nonneg(double x) {
  if (!(x > 0.0)) return 0;
  int e = ilogb(x);
  if (e < -14) e = -14;
  const double r = rint(ldexp(x, 10 - e));   // in [0, 2048]
  return static_cast<uint16_t>(((e + 15) << 10) + static_cast<int>(r) - 1024);
}

// Quantise one group of 32 fp16 values held as 16 dwords (two per dword,
// element 2i in the low half).  Returns the 16 code bytes in codes[4] and
// {scale, min} packed as scale | min << 16 in *meta.
__device__ __forceinline__ void quant_group32(const uint32_t in[16], uint32_t codes[4],
                                              uint32_t* meta) {
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = h2f(static_cast<uint16_t>(in[i] & 0xFFFFu));
    const float b = h2f(static_cast<uint16_t>(in[i] >> 16));
    mn = fminf(mn, fminf(a, b));
    mx = fmaxf(mx, fmaxf(a, b));
  }
  const double m = static_cast<double>(mn) + 0.0;    // canonical +0 for a zero min
  const uint16_t s_bits = d2h_rne_nonneg((static_cast<double>(mx) - m) / 15.0);
  const double s = static_cast<double>(h2f(s_bits));
  const _Float16 m_h = static_cast<_Float16>(static_cast<float>(m));
  *meta = static_cast<uint32_t>(s_bits) |
          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, m_h)) << 16);
#pragma unroll
  for (int w = 0; w < 4; ++w) codes[w] = 0;
  if (s_bits == 0) return;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const double x = static_cast<double>(h2f(static_cast<uint16_t>(in[i] >> (16 * h))));
      double c = rint((x - m) / s);
      c = c < 0.0 ? 0.0 : (c > 15.0 ? 15.0 : c);
      const int e = 2 * i + h;                 // element index in the group
      codes[e >> 3] |= static_cast<uint32_t>(c) << (4 * (e & 7));
    }
  }
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

}  // namespace hq

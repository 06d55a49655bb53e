// Device-side helpers shared by the gfx950 kernels of libhq.
//
// The group rule (per token, per 32 consecutive head_dim elements), for
// b-bit codes (b = 4 for K4V4; 2 and 8 for the other strict low-bit caches):
// min m, max M, scale s = fp16_rne((M - m) / (2^b - 1)), code =
// clamp(rne((x - m)/s), 0, 2^b - 1), all codes 0 when s == 0; 8/b codes per
// byte, the lower element in the lower bits.  The scale is decided in fp64,
// and so is every code whose float32 estimate is close to a half-integer:
// x - m and M - m are exact there (fp16 differences need at most 41
// significant bits), and the single correctly-rounded fp64 division cannot
// move a quotient across a half-integer boundary or an fp16 rounding
// midpoint (the divisors are at most 255), so the codes equal the
// exact-arithmetic definition (exact_code below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int kD = 128;        // head_dim
constexpr int kGroup = 32;     // elements per quantisation group
constexpr int kRowBytes = kD / 2;        // packed 4-bit code bytes per token
template <int kBits>
constexpr int row_bytes() { return kD * kBits / 8; }   // packed b-bit code bytes per token
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

// The code of one element, x in [m, M], by the exact rule.  A float32
// quotient (x - m) / s decides it unless the quotient lies within 5e-4 of a
// half-integer: x - m, 1/s and their product are each rounded once, so its
// relative error is below 2^-21 and its absolute error below 1e-4 for every
// quotient up to 2^b, where the clamp does not already decide.  Near a
// half-integer the fp64 division (exact decision) is taken instead.
__device__ __forceinline__ uint32_t exact_code(float x, float mf, float rf, double m, double s, float qmax) {
  const float q = (x - mf) * rf;
  float c = rintf(q);
  if (q <= qmax + 1.0f && fabsf(q - floorf(q) - 0.5f) <= 5e-4f)
    c = static_cast<float>(rint((static_cast<double>(x) - m) / s));
  return static_cast<uint32_t>(fminf(fmaxf(c, 0.0f), qmax));
}

// Quantise one group of 32 fp16 values held as 16 dwords (two per dword,
// element 2i in the low half) to b-bit codes.  Returns the 4 b code bytes in
// codes[kBits] (element e at bits b e .. of the little-endian group) and
// {scale, min} packed as scale | min << 16 in *meta.
template <int kBits = 4>
__device__ __forceinline__ void quant_group32(const uint32_t in[16], uint32_t codes[kBits],
                                              uint32_t* meta) {
  constexpr int kQmax = (1 << kBits) - 1;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = h2f(static_cast<uint16_t>(in[i] & 0xFFFFu));
    const float b = h2f(static_cast<uint16_t>(in[i] >> 16));
    mn = fminf(mn, fminf(a, b));
    mx = fmaxf(mx, fmaxf(a, b));
  }
  const double m = static_cast<double>(mn) + 0.0;    // canonical +0 for a zero min
  const uint16_t s_bits = d2h_rne_nonneg((static_cast<double>(mx) - m) / static_cast<double>(kQmax));
  const double s = static_cast<double>(h2f(s_bits));
  const _Float16 m_h = static_cast<_Float16>(static_cast<float>(m));
  *meta = static_cast<uint32_t>(s_bits) |
          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, m_h)) << 16);
#pragma unroll
  for (int w = 0; w < kBits; ++w) codes[w] = 0;
  if (s_bits == 0) return;
  const float rf = 1.0f / h2f(s_bits);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float x = h2f(static_cast<uint16_t>(in[i] >> (16 * h)));
      const uint32_t c = exact_code(x, mn, rf, m, s, static_cast<float>(kQmax));
      const int e = 2 * i + h;                 // element index in the group
      codes[(kBits * e) >> 5] |= c << ((kBits * e) & 31);
    }
  }
}

// Quantise one group and store its codes (4 b bytes at `dst`, 8-byte
// aligned) and {scale, min} word.
template <int kBits>
__device__ __forceinline__ void quant_store_group(const uint32_t in[16], uint8_t* dst, uint32_t* meta_dst) {
  uint32_t codes[kBits], meta;
  quant_group32<kBits>(in, codes, &meta);
  if constexpr (kBits == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(codes[0], codes[1]);
  } else {
#pragma unroll
    for (int w = 0; w < kBits; w += 4)
      *reinterpret_cast<uint4*>(dst + 4 * w) = make_uint4(codes[w], codes[w + 1], codes[w + 2], codes[w + 3]);
  }
  *meta_dst = meta;
}

// Width chosen at run time (K and V may differ): 2, 4 or 8 bits.
__device__ __forceinline__ void quant_store_group_bits(int bits, const uint32_t in[16], uint8_t* dst,
                                                       uint32_t* meta_dst) {
  if (bits == 2) quant_store_group<2>(in, dst, meta_dst);
  else if (bits == 8) quant_store_group<8>(in, dst, meta_dst);
  else quant_store_group<4>(in, dst, meta_dst);
}

// The same rule for a group spread over the four lanes of a lane quad, 8
// values each (quad lane i holds elements 8i .. 8i+7 of the group, two per
// dword, the lower element in the low half).  The min and max are reduced
// across the quad, so every lane of the wave must make the call.  Returns
// this lane's 8 codes in the low 8 b bits (element 8i + j at bit b j), and
// the group's {scale, min} word in *meta.
__device__ __forceinline__ uint64_t quant_quad8(const uint4 v, int bits, uint32_t* meta) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
    const float b = h2f(static_cast<uint16_t>(w[i] >> 16));
    mn = fminf(mn, fminf(a, b));
    mx = fmaxf(mx, fmaxf(a, b));
  }
  mn = fminf(mn, __shfl_xor(mn, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  mn = fminf(mn, __shfl_xor(mn, 2));
  mx = fmaxf(mx, __shfl_xor(mx, 2));
  const double qmax = static_cast<double>((1 << bits) - 1);
  const double m = static_cast<double>(mn) + 0.0;    // canonical +0 for a zero min
  const uint16_t s_bits = d2h_rne_nonneg((static_cast<double>(mx) - m) / qmax);
  const double s = static_cast<double>(h2f(s_bits));
  const _Float16 m_h = static_cast<_Float16>(static_cast<float>(m));
  *meta = static_cast<uint32_t>(s_bits) |
          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, m_h)) << 16);
  uint64_t codes = 0;
  if (s_bits == 0) return codes;
  const float rf = 1.0f / h2f(s_bits);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = h2f(static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1))));
    const uint32_t c = exact_code(x, mn, rf, m, s, static_cast<float>(qmax));
    codes |= static_cast<uint64_t>(c) << (bits * j);
  }
  return codes;
}

// Store a lane's 8 b-bit codes (b bytes) at `dst`, b-byte aligned.
__device__ __forceinline__ void store_codes8(uint8_t* dst, uint64_t codes, int bits) {
  if (bits == 2) *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(codes);
  else if (bits == 8) *reinterpret_cast<uint2*>(dst) =
      make_uint2(static_cast<uint32_t>(codes), static_cast<uint32_t>(codes >> 32));
  else *reinterpret_cast<uint32_t*>(dst) = static_cast<uint32_t>(codes);
}

// Flat slot index of K4V4 slot s of unit u: u * cap_q + s, or through the
// unit's page table (32-slot blocks of a shared pool) when the cache is paged.
constexpr int kPageSlots = 32;
__device__ __forceinline__ int64_t k4_slot(const int32_t* pages, int32_t cap_q, int64_t u, int s) {
  if (!pages) return u * cap_q + s;
  return static_cast<int64_t>(pages[u * (cap_q / kPageSlots) + s / kPageSlots]) * kPageSlots +
         (s & (kPageSlots - 1));
}

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Loads of data a launch reads once (the cache regions the decode scan
// streams): the non-temporal policy (nt) keeps them from displacing L2 and
// Infinity Cache contents they would never be read from again.  The decode's
// HBM rate at B = 32, L = 32K went from 5.6 to 6.5 TB/s with them.  Only for
// loads whose lanes cover whole lines in one instruction: a line the next
// instructions still read is not kept under this policy.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

}  // namespace hq

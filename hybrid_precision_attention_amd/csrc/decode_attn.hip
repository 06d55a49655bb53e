// hq_decode_attn for gfx950: split-K flash-decode over the hybrid cache.
//
// One decode query per head attends to a unit's K4V4 tokens, dequantised in
// registers inside the online-softmax scan, and to its FP16 tokens (vertical
// lines, window ring, staging), so no full-precision cache is materialised
// (agihunt digest "HyQuant: Hybrid-Precision Quantization for LLM Attention",
// decode paragraph; HyQuant README, Overview item 3: online softmax over
// quantised blocks).
//
// Work decomposition.  Grid = (splits, units).  The first nsplit_q
// workgroups of a unit scan contiguous ranges of its K4V4 slots, the rest scan
// ranges of the FP16 sequence (vertical lines, then window slots, then
// staging).  Each workgroup has four waves that take 32-token blocks in turn;
// the waves' (max, sum, output) triples are merged in LDS into one partial
// record, and the last workgroup of the unit to arrive (an atomic counter in
// the workspace) merges the unit's records by log-sum-exp and writes out/lse.
//
// Per 32-token block a wave runs, for the G query heads of the unit (padded
// to 16):  S = K Q^T with two 16-token tiles x four k-steps of
// v_mfma_f32_16x16x32_f16, an online softmax in base 2, and O^T += V^T P^T
// with eight MFMAs (one per group of 16 output dims).  The contraction order
// inside an MFMA is free, so operands are laid out for the loads:
//  * K tile (A operand, M = tokens): lane (t, j) loads the 16 code bytes of
//    group j of token t with one 128-bit load; k-step kk uses its dword kk.
//    The nibble unpack yields element order {0,4,1,5,2,6,3,7}, and Q (the B
//    operand) is permuted the same way once per wave.
//  * V^T (A operand, M = dims, K = tokens): lane (r, j) loads dword r (dims
//    8r..8r+7) of the eight tokens it owns and MFMA i uses nibble i, so the
//    wave's loads still cover whole 64-byte code rows.
//  * P^T (B operand) is the softmax of the lane's own S values: the tokens a
//    lane holds after QK are exactly the tokens its PV k-slice contracts.
//  * O^T (D): lane (head n, j) ends with dims 32j..32j+31 of head n.
// Nibbles become fp16 by OR-ing them under the exponent of 1024 (0x6400),
// subtracting 1024 (exact) and one fused multiply-add with {scale, min}.
#include <hip/hip_runtime.h>
#include <math.h>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 32;
constexpr int kPart = 132;          // floats per partial record: m, l, pad, pad, o[128]
constexpr uint32_t kMagic = 0x64006400u;

struct DecodeArgs {
  hq_cache c;
  const uint16_t* q;
  uint16_t* out;
  float* lse;
  float* part;
  int32_t* counters;
  int32_t Hq, Hkv, G, W, cap_q, cap_vl, cap_stg;
  int32_t n_win;
  int32_t nsplit_q, nsplit_f;
  float c2;                         // log2(e) / sqrt(d)
};

__device__ __forceinline__ half8_t as_half8(uint4 v) { return __builtin_bit_cast(half8_t, v); }
__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

// four packed fp16 pairs -> half8
__device__ __forceinline__ half8_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return as_half8(make_uint4(a, b, c, d));
}

// (1024 + code) pair -> code * scale + min, rounded once to fp16
__device__ __forceinline__ uint32_t dq_pair(uint32_t biased, half2_t s, half2_t m) {
  const half2_t c = as_half2(biased) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
  return as_u32(__builtin_elementwise_fma(c, s, m));
}

// Eight nibbles of one K group -> A-operand half8 in element order
// {0,4,1,5,2,6,3,7}; meta = scale | min << 16.
__device__ __forceinline__ half8_t dq_k8(uint32_t w, uint32_t meta) {
  const half2_t s = as_half2((meta & 0xFFFFu) * 0x10001u);
  const half2_t m = as_half2((meta >> 16) * 0x10001u);
  const uint32_t p0 = (w & 0x000F000Fu) | kMagic;
  const uint32_t p1 = ((w >> 4) & 0x000F000Fu) | kMagic;
  const uint32_t p2 = ((w >> 8) & 0x000F000Fu) | kMagic;
  const uint32_t p3 = ((w >> 12) & 0x000F000Fu) | kMagic;
  return pack4(dq_pair(p0, s, m), dq_pair(p1, s, m), dq_pair(p2, s, m), dq_pair(p3, s, m));
}

__device__ __forceinline__ float4_t mfma(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max_over_j(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Online-softmax state of one wave: lane (head n, j).
struct SoftState {
  float m;                          // running max of raw scores q.k (same for all j)
  float l;                          // this lane's share of the running denominator
  float4_t o[8];                    // O^T: o[i][r] = head n, dim 32j + 8r + i
};

// Fold one 32-token block of raw scores s[8] (tokens 4j+r and 16+4j+r, -inf
// when masked) into the state; returns the B operand P^T for the PV MFMAs.
__device__ __forceinline__ half8_t softmax_block(SoftState& st, const float s[8], float c2) {
  float bm = s[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) bm = fmaxf(bm, s[e]);
  bm = wave_max_over_j(bm);
  const float m_new = fmaxf(st.m, bm);
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float alpha = exp2f((st.m - m_use) * c2);
  const float nmc = -m_use * c2;
  float p[8];
  float ps = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2f(fmaf(s[e], c2, nmc));
    ps += p[e];
  }
  st.l = fmaf(st.l, alpha, ps);
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[i] *= alpha;
  st.m = m_new;
  half8_t pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) pb[e] = static_cast<_Float16>(p[e]);
  return pb;
}

// Raw loads of one K4V4 block for one lane.
struct K4Raw {
  uint4 ka, kb;                     // code bytes of group j of tokens tb+t and tb+16+t
  uint32_t kma, kmb;                // their {scale, min}
  uint32_t vc[8];                   // dword r of the V code rows of the lane's 8 tokens
  uint32_t vm[8];                   // {scale, min} of group r/4 of those tokens
};

__device__ __forceinline__ int k4_token(int tb, int j, int e) {
  return tb + (e < 4 ? 4 * j + e : 16 + 4 * j + (e - 4));
}

__device__ __forceinline__ void load_k4(K4Raw& r, const uint8_t* kq, const uint32_t* kmeta,
                                        const uint8_t* vq, const uint32_t* vmeta, int tb,
                                        int nq, int n, int j) {
  const int ta = min(tb + n, nq - 1);
  const int tbb = min(tb + 16 + n, nq - 1);
  r.ka = ld16(kq + static_cast<int64_t>(ta) * kRowBytes + 16 * j);
  r.kb = ld16(kq + static_cast<int64_t>(tbb) * kRowBytes + 16 * j);
  r.kma = kmeta[static_cast<int64_t>(ta) * kMetaWords + j];
  r.kmb = kmeta[static_cast<int64_t>(tbb) * kMetaWords + j];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = min(k4_token(tb, j, e), nq - 1);
    r.vc[e] = *reinterpret_cast<const uint32_t*>(vq + static_cast<int64_t>(t) * kRowBytes + 4 * n);
    r.vm[e] = vmeta[static_cast<int64_t>(t) * kMetaWords + (n >> 2)];
  }
}

__device__ __forceinline__ void compute_k4(SoftState& st, const K4Raw& r, const half8_t qb[4],
                                           int tb, int nq, int j, float c2) {
  float4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
  const uint32_t ka[4] = {r.ka.x, r.ka.y, r.ka.z, r.ka.w};
  const uint32_t kb[4] = {r.kb.x, r.kb.y, r.kb.z, r.kb.w};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    sa = mfma(dq_k8(ka[kk], r.kma), qb[kk], sa);
    sb = mfma(dq_k8(kb[kk], r.kmb), qb[kk], sb);
  }
  float s[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[e] = (tb + 4 * j + e < nq) ? sa[e] : -INFINITY;
    s[4 + e] = (tb + 16 + 4 * j + e < nq) ? sb[e] : -INFINITY;
  }
  const half8_t pb = softmax_block(st, s, c2);

  // V^T operands: token pairs (2p, 2p+1) interleaved so one and_or gives a
  // (1024 + code) fp16 pair for both tokens
  uint32_t xlo[4], xhi[4];
  half2_t sp[4], mp[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    xlo[p] = __builtin_amdgcn_perm(r.vc[2 * p + 1], r.vc[2 * p], 0x05040100u);
    xhi[p] = __builtin_amdgcn_perm(r.vc[2 * p + 1], r.vc[2 * p], 0x07060302u);
    sp[p] = as_half2(__builtin_amdgcn_perm(r.vm[2 * p + 1], r.vm[2 * p], 0x05040100u));
    mp[p] = as_half2(__builtin_amdgcn_perm(r.vm[2 * p + 1], r.vm[2 * p], 0x07060302u));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sh = 4 * (i & 3);
    uint32_t v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t x = (i < 4) ? xlo[p] : xhi[p];
      v[p] = dq_pair(((x >> sh) & 0x000F000Fu) | kMagic, sp[p], mp[p]);
    }
    st.o[i] = mfma(pack4(v[0], v[1], v[2], v[3]), pb, st.o[i]);
  }
}

// FP16 token v of a unit's FP16 sequence: vertical lines, window, staging.
__device__ __forceinline__ const uint16_t* f16_row(const uint16_t* vl, const uint16_t* win,
                                                   const uint16_t* stg, int v, int nvl,
                                                   int nwin) {
  if (v < nvl) return vl + static_cast<int64_t>(v) * kD;
  if (v < nvl + nwin) return win + static_cast<int64_t>(v - nvl) * kD;
  return stg + static_cast<int64_t>(v - nvl - nwin) * kD;
}

__device__ __forceinline__ void process_f16(SoftState& st, const half8_t qn[4],
                                            const uint16_t* kvl, const uint16_t* kwin,
                                            const uint16_t* kstg, const uint16_t* vvl,
                                            const uint16_t* vwin, const uint16_t* vstg, int tb,
                                            int nvl, int nwin, int nf, int n, int j, float c2) {
  const int ta = min(tb + n, nf - 1);
  const int tbb = min(tb + 16 + n, nf - 1);
  const uint16_t* ra = f16_row(kvl, kwin, kstg, ta, nvl, nwin) + 32 * j;
  const uint16_t* rb = f16_row(kvl, kwin, kstg, tbb, nvl, nwin) + 32 * j;
  uint4 ka[4], kb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    ka[kk] = ld16(ra + 8 * kk);
    kb[kk] = ld16(rb + 8 * kk);
  }
  uint4 vr[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = min(k4_token(tb, j, e), nf - 1);
    vr[e] = ld16(f16_row(vvl, vwin, vstg, t, nvl, nwin) + 8 * n);
  }
  float4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    sa = mfma(as_half8(ka[kk]), qn[kk], sa);
    sb = mfma(as_half8(kb[kk]), qn[kk], sb);
  }
  float s[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s[e] = (tb + 4 * j + e < nf) ? sa[e] : -INFINITY;
    s[4 + e] = (tb + 16 + 4 * j + e < nf) ? sb[e] : -INFINITY;
  }
  const half8_t pb = softmax_block(st, s, c2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    uint32_t v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a0[4] = {vr[2 * p].x, vr[2 * p].y, vr[2 * p].z, vr[2 * p].w};
      const uint32_t a1[4] = {vr[2 * p + 1].x, vr[2 * p + 1].y, vr[2 * p + 1].z, vr[2 * p + 1].w};
      v[p] = __builtin_amdgcn_perm(a1[i >> 1], a0[i >> 1], sel);
    }
    st.o[i] = mfma(pack4(v[0], v[1], v[2], v[3]), pb, st.o[i]);
  }
}

__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_o[kWaves][16][kD + 4];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, j = lane >> 4;
  const int64_t u = blockIdx.y;
  const int split = blockIdx.x;
  const int nsplit = a.nsplit_q + a.nsplit_f;
  const int G = a.G;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * G;
  const float c2 = a.c2;

  // this lane's slice of the query: head h0 + n, dims 32j..32j+31
  uint4 qraw[4];
  if (n < G) {
    const uint16_t* qp = a.q + (b * a.Hq + h0 + n) * kD + 32 * j;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qraw[kk] = ld16(qp + 8 * kk);
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qraw[kk] = make_uint4(0, 0, 0, 0);
  }

  SoftState st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[i] = (float4_t){0.f, 0.f, 0.f, 0.f};

  if (split < a.nsplit_q) {
    const int nq = min(a.c.n_q[u], a.cap_q);
    const int nblk = (nq + kBlk - 1) / kBlk;
    const int b0 = static_cast<int>(static_cast<int64_t>(nblk) * split / a.nsplit_q);
    const int b1 = static_cast<int>(static_cast<int64_t>(nblk) * (split + 1) / a.nsplit_q);
    half8_t qb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const half8_t nat = as_half8(qraw[kk]);
      qb[kk] = __builtin_shufflevector(nat, nat, 0, 4, 1, 5, 2, 6, 3, 7);
    }
    const uint8_t* kq = a.c.kq + u * a.cap_q * kRowBytes;
    const uint8_t* vq = a.c.vq + u * a.cap_q * kRowBytes;
    const uint32_t* kmeta = reinterpret_cast<const uint32_t*>(a.c.kq_meta) + u * a.cap_q * kMetaWords;
    const uint32_t* vmeta = reinterpret_cast<const uint32_t*>(a.c.vq_meta) + u * a.cap_q * kMetaWords;
    int blk = b0 + wave;
    if (blk < b1) {
      K4Raw cur;
      load_k4(cur, kq, kmeta, vq, vmeta, blk * kBlk, nq, n, j);
      for (; blk < b1; blk += kWaves) {
        K4Raw nxt;
        const int nb = blk + kWaves;
        if (nb < b1) load_k4(nxt, kq, kmeta, vq, vmeta, nb * kBlk, nq, n, j);
        compute_k4(st, cur, qb, blk * kBlk, nq, j, c2);
        cur = nxt;
      }
    }
  } else {
    const int sf = split - a.nsplit_q;
    const int nvl = min(a.c.n_vl[u], a.cap_vl);
    const int nst = min(a.c.n_stg[u], a.cap_stg);
    const int nwin = a.n_win;
    const int nf = nvl + nwin + nst;
    const int nblk = (nf + kBlk - 1) / kBlk;
    const int b0 = static_cast<int>(static_cast<int64_t>(nblk) * sf / a.nsplit_f);
    const int b1 = static_cast<int>(static_cast<int64_t>(nblk) * (sf + 1) / a.nsplit_f);
    half8_t qn[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qn[kk] = as_half8(qraw[kk]);
    const uint16_t* kvl = a.c.kvl + u * a.cap_vl * kD;
    const uint16_t* vvl = a.c.vvl + u * a.cap_vl * kD;
    const uint16_t* kwin = a.W > 0 ? a.c.kwin + u * a.W * kD : nullptr;
    const uint16_t* vwin = a.W > 0 ? a.c.vwin + u * a.W * kD : nullptr;
    const uint16_t* kstg = a.c.kstg + u * a.cap_stg * kD;
    const uint16_t* vstg = a.c.vstg + u * a.cap_stg * kD;
    for (int blk = b0 + wave; blk < b1; blk += kWaves)
      process_f16(st, qn, kvl, kwin, kstg, vvl, vwin, vstg, blk * kBlk, nvl, nwin, nf, n, j, c2);
  }

  // wave -> LDS
  float lt = st.l;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (j == 0) {
    s_m[wave][n] = st.m;
    s_l[wave][n] = lt;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[wave][n][32 * j + 8 * r + i] = st.o[i][r];
  __syncthreads();

  // workgroup partial record
  float* rec0 = a.part + (u * nsplit + split) * static_cast<int64_t>(G) * kPart;
  for (int idx = tid; idx < G * kD; idx += kThreads) {
    const int g = idx >> 7, dim = idx & (kD - 1);
    float mm = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, s_m[w][g]);
    float o = 0.0f, ls = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f((s_m[w][g] - mm) * c2);
        o = fmaf(f, s_o[w][g][dim], o);
        ls = fmaf(f, s_l[w][g], ls);
      }
    }
    float* rec = rec0 + g * kPart;
    rec[4 + dim] = o;
    if (dim == 0) {
      rec[0] = mm;
      rec[1] = ls;
    }
  }

  // arrival counter: the last workgroup of the unit merges all records
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(a.counters + u, 1);
    s_last = (old == nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const float* recu = a.part + u * nsplit * static_cast<int64_t>(G) * kPart;
  for (int idx = tid; idx < G * kD; idx += kThreads) {
    const int g = idx >> 7, dim = idx & (kD - 1);
    float mm = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mm = fmaxf(mm, recu[(static_cast<int64_t>(s) * G + g) * kPart]);
    float o = 0.0f, ls = 0.0f;
    if (mm != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float* rec = recu + (static_cast<int64_t>(s) * G + g) * kPart;
        const float f = exp2f((rec[0] - mm) * c2);
        o = fmaf(f, rec[4 + dim], o);
        ls = fmaf(f, rec[1], ls);
      }
    }
    const float res = ls > 0.0f ? o / ls : 0.0f;
    a.out[(b * a.Hq + h0 + g) * kD + dim] =
        __builtin_bit_cast(uint16_t, static_cast<_Float16>(res));
    if (dim == 0 && a.lse)
      a.lse[b * a.Hq + h0 + g] = ls > 0.0f ? (mm * c2 + log2f(ls)) * 0.69314718055994531f : -INFINITY;
  }
  if (tid == 0) a.counters[u] = 0;
}

}  // namespace

hipError_t launch_decode(const hq_dims& d, const hq_cache& c, int32_t L, const DecodePlan& plan,
                         const uint16_t* q, uint16_t* out, float* lse, void* ws, hipStream_t s) {
  DecodeArgs a;
  a.c = c;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.counters = reinterpret_cast<int32_t*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + decode_counter_bytes(d));
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.W = d.W;
  a.cap_q = d.cap_q;
  a.cap_vl = d.cap_vl;
  a.cap_stg = d.cap_stg;
  a.n_win = plan.n_win;
  a.nsplit_q = plan.nsplit_q;
  a.nsplit_f = plan.nsplit_f;
  a.c2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d.d)));
  (void)L;
  dim3 grid(plan.nsplit_q + plan.nsplit_f, d.B * d.Hkv);
  hipLaunchKernelGGL(decode_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hq

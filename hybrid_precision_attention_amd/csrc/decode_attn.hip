// hq_decode_attn for gfx950: split-K flash-decode over the hybrid cache.
//
// One decode query per head attends to a unit's K4V4 tokens, dequantised in
// registers inside the online-softmax scan, and to its FP16 tokens (vertical
// lines, window ring, staging), so no full-precision cache is materialised
// (agihunt digest "HyQuant: Hybrid-Precision Quantization for LLM Attention",
// decode paragraph; HyQuant README, Overview item 3: online softmax over
// quantised blocks).
//
// Work decomposition.  Grid = (splits, units).  A unit's work is its K4V4
// slots in 32-token blocks and its FP16 sequence (vertical lines, window
// slots, staging) in 32-token blocks; of the unit's nsplit * 4 waves, each
// takes a contiguous range of K4V4 blocks and every (nsplit * 4)-th FP16
// block, sized so that every wave streams about the same bytes (wave_work).
// Workgroups are four waves, one per SIMD; the host's split plan puts one
// workgroup on each CU for the G <= 4 scan at 4- and 8-bit widths and up to
// two for the others (the scan's register count allows two).  Each workgroup
// merges its four waves' (max, sum, output) states through LDS into one
// partial record; the last workgroup of the unit to arrive (an atomic
// counter in the workspace) merges the unit's records by log-sum-exp and
// writes out/lse.
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
//  * V^T (A operand, M = dims, K = tokens): lane (r, j) needs dword r (dims
//    8r..8r+7) of the eight tokens it owns, and MFMA i uses nibble i.  The
//    block's V codes and all its {scale, min} words arrive with 128/64-bit
//    loads and are transposed through a per-wave LDS staging area: six vector
//    memory instructions per block instead of twenty.
//  * P^T (B operand) is the softmax of the lane's own S values: the tokens a
//    lane holds after QK are exactly the tokens its PV k-slice contracts.
//  * O^T (D): lane (head n, j) ends with dims 32j..32j+31 of head n.
// Nibbles become fp16 by OR-ing them under the exponent of 1024 (0x6400):
// the low nibble of a byte gives 1024 + c, the high nibble (masked in place)
// 1024 + 16c; subtracting 1024 is exact, and one fused multiply-add with
// {scale, min} (or {scale/16, min}) finishes the dequantisation.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>
#include <type_traits>

#include "hq_device.h"
#include "hq_launch.h"

namespace hq {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 32;
constexpr int kPart = kPartFloatsPerRecord;   // floats per partial record: m, l, pad, pad, o[128]
constexpr int kFoldItems = 2;       // outputs (head, 4 dims) per thread: G * 32 <= 2 * kThreads
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3 for raw 32-bit loads (gfx9 family)
constexpr int kSc1 = 16;            // cache-policy bit sc1 of a buffer load: device-scope coherent

struct DecodeArgs {
  hq_cache c;
  const uint16_t* q;
  uint16_t* out;
  float* lse;
  float* part;
  int32_t* counters;
  int32_t Hq, Hkv, G, W, cap_q, cap_vl, cap_stg;
  int32_t n_win;
  const int32_t* L_seq;             // [B] per-sequence query positions (ragged batch), or null
  int32_t L_max;
  int32_t nsplit;                   // workgroups per unit
  float c2;                         // log2(e) / sqrt(d)
  float slack;                      // 8 / c2: how far a block's max may pass the running reference
  // decode step with its staging merge (hq_decode_step): the new token's
  // rows take the place of the staging slot, and the unit's last workgroup
  // moves them into the ring afterwards; null for a plain decode
  const uint16_t* k_new;            // [B][Hkv][d]
  const uint16_t* v_new;
  const uint8_t* evict_is_vl;       // [B][Hkv] or null
};

__device__ __forceinline__ half8_t as_half8(uint4 v) { return __builtin_bit_cast(half8_t, v); }

// The staging merge of a decode step at position t, run by one wave of the
// unit's last workgroup once every workgroup of the unit has finished its
// scan (so nothing reads the ring any more): the token leaving the window
// (position t - W; with no window the new token itself) is quantised into
// the next K4V4 slot, or copied to the vertical-line region when flagged,
// and the new token takes its ring slot t mod W.  Lanes 0-15 carry the K
// row, 16-31 the V row, 16 bytes each; a quantisation group is a lane quad.
// step_load issues every load of the merge, so that they are in flight
// while the workgroup folds the records; step_store finishes it.
struct StepIn {
  uint4 fresh, old;
  int nq, nvl;
  bool flagged;
};

__device__ __forceinline__ StepIn step_load(const DecodeArgs& a, int64_t u, int t, int lane) {
  const bool mover = lane < 32;
  const int kv = (lane >> 4) & 1, part = lane & 15;
  const int W = a.W;
  const int ev = t - W;
  const uint16_t* win = W > 0 ? (kv ? a.c.vwin : a.c.kwin) + (u * W + t % W) * kD + 8 * part : nullptr;
  StepIn in;
  in.fresh = mover ? ld16((kv ? a.v_new : a.k_new) + u * kD + 8 * part) : make_uint4(0, 0, 0, 0);
  in.old = (mover && win && ev >= 0) ? ld16(win) : make_uint4(0, 0, 0, 0);
  in.nq = a.c.n_q[u];
  in.nvl = a.c.n_vl[u];
  in.flagged = a.evict_is_vl && a.evict_is_vl[u] != 0;
  return in;
}

template <int kKB, int kVB>
__device__ __forceinline__ void step_store(const DecodeArgs& a, int64_t u, int t, int lane, const StepIn& in) {
  const bool mover = lane < 32;
  const int kv = (lane >> 4) & 1, part = lane & 15;
  const int W = a.W;
  const int ev = t - W;
  uint16_t* win = W > 0 ? (kv ? a.c.vwin : a.c.kwin) + (u * W + t % W) * kD + 8 * part : nullptr;
  const int nq = in.nq, nvl = in.nvl;
  if (ev >= 0) {
    const uint4 evv = W > 0 ? in.old : in.fresh;
    const bool to_vl = in.flagged && nvl < a.cap_vl;
    if (to_vl) {
      if (mover) st16((kv ? a.c.vvl : a.c.kvl) + (u * a.cap_vl + nvl) * kD + 8 * part, evv);
      if (lane == 0) {
        a.c.vl_pos[u * a.cap_vl + nvl] = ev;
        a.c.n_vl[u] = nvl + 1;
      }
    } else if (nq < a.cap_q) {
      const int bits = kv ? kVB : kKB;
      uint32_t meta;
      const uint64_t codes = quant_quad8(evv, bits, &meta);
      const int64_t slot = k4_slot(a.c.k4_pages, a.cap_q, u, nq);
      if (mover) {
        store_codes8((kv ? a.c.vq : a.c.kq) + slot * (kD * bits / 8) + bits * part, codes, bits);
        if ((part & 3) == 0)
          reinterpret_cast<uint32_t*>(kv ? a.c.vq_meta : a.c.kq_meta)[slot * kMetaWords + (part >> 2)] = meta;
      }
      if (lane == 0) {
        a.c.q_pos[slot] = ev;
        a.c.n_q[u] = nq + 1;
      }
    }
  }
  // the leaving token's read (in step_load) completes before its slot is
  // overwritten: the empty statement consumes the loaded value, so the
  // compiler waits for that load (and not for the younger stores)
  if (win && mover) {
    asm volatile("" : : "v"(in.old.x), "v"(in.old.w));
    st16(win, in.fresh);
  }
}

// Valid window slots of sequence b: min(W, L) at its own position L in a
// ragged batch (clamped to [0, L_max]), else the batch's common count.
__device__ __forceinline__ int unit_n_win(const DecodeArgs& a, int64_t b) {
  if (!a.L_seq) return a.n_win;
  const int L = min(max(a.L_seq[b], 0), a.L_max);
  return min(a.W, L);
}
__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t as_u32(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ half8_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return as_half8(make_uint4(a, b, c, d));
}

// Unpack constants held in VGPRs: gfx950 VOP3 encodings take no literal, so
// with the masks in registers (x & mask) | magic is one v_and_or_b32.
struct Masks {
  uint32_t lo, hi, magic;
};

__device__ __forceinline__ Masks make_masks() {
  Masks k;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(k.lo));
  asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(k.hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
  return k;
}

// biased fp16 pair (1024 + k) -> k * s + m, rounded once
__device__ __forceinline__ uint32_t dq_pair(uint32_t biased, half2_t s, half2_t m) {
  const half2_t c = as_half2(biased) - (half2_t){(_Float16)1024.0f, (_Float16)1024.0f};
  return as_u32(__builtin_elementwise_fma(c, s, m));
}

__device__ __forceinline__ half2_t sixteenth(half2_t s) {
  return s * (half2_t){(_Float16)0.0625f, (_Float16)0.0625f};
}

// Eight nibbles of one K group -> A-operand half8 in element order
// {0,4,1,5,2,6,3,7}; s/s16/m are the group's scale, scale/16 and min.
__device__ __forceinline__ half8_t dq_k8(uint32_t w, half2_t s, half2_t s16, half2_t m,
                                        const Masks& k) {
  const uint32_t w8 = w >> 8;
  return pack4(dq_pair((w & k.lo) | k.magic, s, m), dq_pair((w & k.hi) | k.magic, s16, m),
               dq_pair((w8 & k.lo) | k.magic, s, m), dq_pair((w8 & k.hi) | k.magic, s16, m));
}

__device__ __forceinline__ float4_t mfma(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The running reference m of an online softmax moves only when a block's
// maximum exceeds it by `slack` (raw-score units, 8 / c2: a factor of 2^8 in
// probability), so every p = 2^((s - m) c2) stays at most 256, which the
// fp16 P operand and the fp32 sums hold with the same relative precision as
// p <= 1, and the rescale of the accumulators runs a few times per scan
// rather than at every new maximum.  The first block of a scan only sets m
// (the accumulators are still zero).  Any reference gives the same result:
// the partial records carry it, and the merges rescale by it.
template <typename Scale>
__device__ __forceinline__ void rescale_on_growth(float& m, float bm, float slack, float c2, Scale&& scale) {
  const bool grow = bm > m + slack;
  if (__any(grow)) {
    const float m_new = grow ? bm : m;
    if (__any(grow && m != -INFINITY)) scale(grow ? __builtin_amdgcn_exp2f((m - m_new) * c2) : 1.0f);
    m = m_new;
  }
}

// Online-softmax state of one wave: lane (head n, j).
struct SoftState {
  float m;                          // running max of raw scores q.k (same for all j)
  float l;                          // this lane's share of the running denominator
  float4_t o[8];                    // O^T: o[i][r] = head n, dim 32j + 8r + i
};

// Fold one 32-token block of raw scores s[8] (tokens 4j+r and 16+4j+r, -inf
// when masked) into the state; returns the B operand P^T for the PV MFMAs.
// The accumulator is rescaled only when some head's running max grew.
__device__ __forceinline__ half8_t softmax_block(SoftState& st, const float s[8], float c2, float slack) {
  float bm = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                   fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  {  // max over the four j-lanes of the head (lanes l^16, l^32)
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
  }
  rescale_on_growth(st.m, bm, slack, c2, [&](float alpha) {
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.o[i] *= alpha;
  });
  const float nmc = -(st.m == -INFINITY ? 0.0f : st.m) * c2;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c2, nmc));
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  half8_t pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) pb[e] = static_cast<_Float16>(p[e]);
  return pb;
}

// Raw loads of one K4V4 block for one lane: six wide loads per 32 tokens
// (the memory pipeline, not HBM, limits a kernel that issues many narrow ones).
struct K4Raw {
  uint4 ka, kb;                     // K codes, group j of tokens tb+n and tb+16+n
  uint4 va, vb;                     // V codes, 16 bytes of the 2 KB block (row-major)
  uint2 kmw, vmw;                   // two {scale, min} words of K and of V
};

// Per-wave LDS staging of the V codes and all metadata of one block, read
// back transposed: V rows padded to 80 bytes so the eight 4-byte reads of a
// lane column land in distinct banks.
struct K4Stage {
  uint32_t v[32][20];
  uint32_t km[128];                 // word 4t + g: {scale, min} of token t, group g
  uint32_t vm[128];
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int k4_token(int tb, int j, int e) {
  return tb + (e < 4 ? 4 * j + e : 16 + 4 * j + (e - 4));
}

// Rows past the unit's last token are clamped to it, so every address stays
// inside the unit and masked tokens still dequantise to finite values.
template <int kVB = 4, int kKB = 4>
__device__ __forceinline__ void load_k4(K4Raw& r, const uint8_t* kq, const uint32_t* kmeta,
                                        const uint8_t* vq, const uint32_t* vmeta, int tb,
                                        int nq, int lane, int n, int j) {
  // 32-bit byte offsets from the unit's (wave-uniform) base pointers, so the
  // loads take the scalar-base + vector-offset form with no 64-bit math
  const int last = nq - 1;
  const uint32_t oka = static_cast<uint32_t>(min(tb + n, last)) * kRowBytes + 16 * j;
  const uint32_t okb = static_cast<uint32_t>(min(tb + 16 + n, last)) * kRowBytes + 16 * j;
  const uint32_t ova = static_cast<uint32_t>(min(tb + (lane >> 2), last)) * kRowBytes + 16 * (lane & 3);
  const uint32_t ovb = static_cast<uint32_t>(min(tb + 16 + (lane >> 2), last)) * kRowBytes + 16 * (lane & 3);
  const uint32_t om = static_cast<uint32_t>(min(tb + (lane >> 1), last)) * (kMetaWords * 4) + 8 * (lane & 1);
  if constexpr (kKB == 4) {
    r.ka = ld16_stream(kq + oka);
    r.kb = ld16_stream(kq + okb);
  } else {
    // 2-bit K rows are 32 bytes, a group 8 of them (in ka.x, ka.y)
    const int last2 = nq - 1;
    const uint2 a = ld8_stream(kq + static_cast<uint32_t>(min(tb + n, last2)) * row_bytes<2>() + 8 * j);
    const uint2 b = ld8_stream(kq + static_cast<uint32_t>(min(tb + 16 + n, last2)) * row_bytes<2>() + 8 * j);
    r.ka = make_uint4(a.x, a.y, 0u, 0u);
    r.kb = make_uint4(b.x, b.y, 0u, 0u);
  }
  if constexpr (kVB == 4) {
    r.va = ld16_stream(vq + ova);
    r.vb = ld16_stream(vq + ovb);
  } else {
    // 2-bit V rows are 32 bytes: lane l loads half (l & 1) of token l / 2,
    // so one load a lane covers the block (vb is unused)
    const uint32_t ov = static_cast<uint32_t>(min(tb + (lane >> 1), last)) * row_bytes<2>() + 16 * (lane & 1);
    r.va = ld16_stream(vq + ov);
  }
  r.kmw = ld8_stream(reinterpret_cast<const uint8_t*>(kmeta) + om);
  r.vmw = ld8_stream(reinterpret_cast<const uint8_t*>(vmeta) + om);
}

__device__ __forceinline__ void qk_tile(float4_t& acc, uint4 codes, uint32_t meta,
                                        const half8_t qb[4], const Masks& k) {
  const half2_t s = as_half2(__builtin_amdgcn_perm(meta, meta, 0x01000100u));
  const half2_t m = as_half2(__builtin_amdgcn_perm(meta, meta, 0x03020302u));
  const half2_t s16 = sixteenth(s);
  acc = mfma(dq_k8(codes.x, s, s16, m, k), qb[0], acc);
  acc = mfma(dq_k8(codes.y, s, s16, m, k), qb[1], acc);
  acc = mfma(dq_k8(codes.z, s, s16, m, k), qb[2], acc);
  acc = mfma(dq_k8(codes.w, s, s16, m, k), qb[3], acc);
}

__device__ __forceinline__ void compute_k4(SoftState& st, const K4Raw& r, K4Stage& sg,
                                           const half8_t qb[4], const Masks& k, int tb, int nq,
                                           int lane, int n, int j, float c2, float slack) {
  // stage, then read back the transposed operands
  wave_sync();
  *reinterpret_cast<uint4*>(&sg.v[lane >> 2][4 * (lane & 3)]) = r.va;
  *reinterpret_cast<uint4*>(&sg.v[16 + (lane >> 2)][4 * (lane & 3)]) = r.vb;
  *reinterpret_cast<uint2*>(&sg.km[2 * lane]) = r.kmw;
  *reinterpret_cast<uint2*>(&sg.vm[2 * lane]) = r.vmw;
  wave_sync();
  const uint32_t kma = sg.km[4 * n + j];
  const uint32_t kmb = sg.km[64 + 4 * n + j];
  uint32_t vc[8], vm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = k4_token(0, j, e);
    vc[e] = sg.v[t][n];
    vm[e] = sg.vm[4 * t + (n >> 2)];
  }

  float4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
  qk_tile(sa, r.ka, kma, qb, k);
  qk_tile(sb, r.kb, kmb, qb, k);
  float s[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
  if (tb + kBlk > nq) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (tb + 4 * j + e >= nq) s[e] = -INFINITY;
      if (tb + 16 + 4 * j + e >= nq) s[4 + e] = -INFINITY;
    }
  }
  const half8_t pb = softmax_block(st, s, c2, slack);

  // V^T operands: token pairs (2p, 2p+1) interleaved so one and_or gives a
  // biased fp16 pair for both tokens
  uint32_t xl[4], xh[4];
  half2_t sp[4], sp16[4], mp[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    xl[p] = __builtin_amdgcn_perm(vc[2 * p + 1], vc[2 * p], 0x05040100u);
    xh[p] = __builtin_amdgcn_perm(vc[2 * p + 1], vc[2 * p], 0x07060302u);
    sp[p] = as_half2(__builtin_amdgcn_perm(vm[2 * p + 1], vm[2 * p], 0x05040100u));
    mp[p] = as_half2(__builtin_amdgcn_perm(vm[2 * p + 1], vm[2 * p], 0x07060302u));
    sp16[p] = sixteenth(sp[p]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t x = (i < 4) ? xl[p] : xh[p];
      if (i & 2) x >>= 8;
      v[p] = (i & 1) ? dq_pair((x & k.hi) | k.magic, sp16[p], mp[p])
                     : dq_pair((x & k.lo) | k.magic, sp[p], mp[p]);
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

struct F16Rows {
  const uint16_t *kvl, *kwin, *kstg, *vvl, *vwin, *vstg;
  int nvl, nwin, nf;
};

// K rows of one FP16 block: lane (t, j) loads dims 32j..32j+31 of tokens
// tb+t and tb+16+t (natural element order).
__device__ __forceinline__ void load_f16_k(uint4 kr[8], const F16Rows& f, int tb, int n, int j) {
  const int ta = min(tb + n, f.nf - 1);
  const int tbb = min(tb + 16 + n, f.nf - 1);
  const uint16_t* ra = f16_row(f.kvl, f.kwin, f.kstg, ta, f.nvl, f.nwin) + 32 * j;
  const uint16_t* rb = f16_row(f.kvl, f.kwin, f.kstg, tbb, f.nvl, f.nwin) + 32 * j;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kr[kk] = ld16_stream(ra + 8 * kk);
    kr[4 + kk] = ld16_stream(rb + 8 * kk);
  }
}

// One block of fp16 K and V operands (kr: lane (t, j) holds dims 32j ..
// 32j + 31 of tokens t and 16 + t; vr: dims 8n .. 8n + 7 of the lane's eight
// tokens), tokens from `valid` on masked.
__device__ __forceinline__ void f16_compute(SoftState& st, const half8_t qn[4], const uint4 kr[8],
                                            const uint4 vr[8], int valid, int j, float c2, float slack) {
  float4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    sa = mfma(as_half8(kr[kk]), qn[kk], sa);
    sb = mfma(as_half8(kr[4 + kk]), qn[kk], sb);
  }
  float s[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
  if (valid < kBlk) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * j + e >= valid) s[e] = -INFINITY;
      if (16 + 4 * j + e >= valid) s[4 + e] = -INFINITY;
    }
  }
  const half8_t pb = softmax_block(st, s, c2, slack);
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

// V rows of one FP16 block: lane (n, j) loads dims 8n .. 8n + 7 of its
// eight tokens (those its PV k-slice contracts).
__device__ __forceinline__ void load_f16_v(uint4 vr[8], const F16Rows& f, int tb, int n, int j) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = min(k4_token(tb, j, e), f.nf - 1);
    vr[e] = ld16_stream(f16_row(f.vvl, f.vwin, f.vstg, t, f.nvl, f.nwin) + 8 * n);
  }
}

// ---------------------------------------------------------------------------
// Grouped-column path, for G <= 4 query heads per KV head.
//
// The 16 MFMA columns are (head h, group g) pairs, column c = 4h + g.  In the
// QK product the B operand of column c is zero outside group g's 32 dims, so
// every K4V4 code can enter the MFMA as its biased fp16 value (1024 + c, or
// 1024 + 16c for a high nibble, whose query entry is pre-scaled by 1/16) and
// the group's scale and min are applied once per (token, column):
//     q.k_g = s (D - R) + m qs,
// R = 1024 * (sum of the column's operand entries), qs = sum of the group's
// query entries.  A head's four columns are then added inside the lane quad.
// For PV, column c carries P'[t] = s_v[t][g] P[h][t]; output rows of group g
// (the lanes with j = g) collect sum_t (bias + code) P'.  One more MFMA
// against a constant-1024 operand gives the bias (corr) and one against the
// mins gives sum_t m_v[t][g] P[h][t] (mt):
//     O = (o - corr) * (1, or 1/16 for a high nibble) + mt.
// The codes thus need no per-element arithmetic beyond the exponent OR.
// ---------------------------------------------------------------------------
struct GState {
  float m;                          // running max of raw scores of head h (same in the quad, all j)
  float l;                          // this lane's share of the running denominator
  float4_t o[8];                    // o[i][rr]: dims 32j + 8rr + i of head h, used where g == j
  float4_t corr;                    // bias * sum_t P'[t] (every row alike; bias 1024, or 4 for 2-bit V)
  float4_t mt;                      // sum_t m_v[t][j] P[h][t] (every row alike)
  float4_t acc[8];                  // unbiased output of the blocks folded so far (flush_g)
};

// The biased accumulators hold about 1024 sum P' while the output is a
// small fraction of that, so their fp32 rounding error, relative to the
// output, grows with the number of blocks accumulated.  Every kFlushBlocks
// K4V4 blocks they are folded into the unbiased acc, O = (o - corr) (1 or
// 1/16) + mt, and restarted from zero: the error then stays at what a scan
// of that many blocks has, however long the wave's range is.  (With 2-bit
// V codes every dim's operand is 4 + code: the factor is 1, kOdd16 off.)
constexpr int kFlushBlocks = 8;
template <bool kOdd16 = true>
__device__ __forceinline__ void flush_g(GState& st) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float f = (kOdd16 && (i & 1)) ? 0.0625f : 1.0f;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) st.acc[i][rr] += fmaf(st.o[i][rr] - st.corr[rr], f, st.mt[rr]);
    st.o[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
  }
  st.corr = (float4_t){0.f, 0.f, 0.f, 0.f};
  st.mt = (float4_t){0.f, 0.f, 0.f, 0.f};
}

// sum over the lane quad (the four group columns of a head); every lane of
// the quad ends with the same bits
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  return x;
}

__device__ __forceinline__ half8_t k_biased(uint32_t w, const Masks& k) {
  const uint32_t w8 = w >> 8;
  return pack4((w & k.lo) | k.magic, (w & k.hi) | k.magic, (w8 & k.lo) | k.magic, (w8 & k.hi) | k.magic);
}

// 2-bit keys: the eight codes of one 16-bit chunk (code i at bits 2i),
// its low byte in bits 0-7 and its high byte in bits 16-23 of x, as biased
// fp16 pairs (i, 4 + i) in the order {0,4,1,5,2,6,3,7} of k_biased: a code
// goes into mantissa bits 8-9 under the exponent of 4 (exactly 4 + code),
// so the bias is 4 and no query entry needs the 1/16 of a high nibble.
__device__ __forceinline__ half8_t k_biased2(uint32_t x, uint32_t m2, uint32_t mg) {
  return pack4(((x << 8) & m2) | mg, ((x << 6) & m2) | mg, ((x << 4) & m2) | mg, ((x << 2) & m2) | mg);
}

// Online softmax of one block of raw scores s[8] into the grouped state;
// p[8] gets the block's probabilities.
__device__ __forceinline__ void softmax_g(GState& st, const float s[8], float c2, float slack, float p[8]) {
  float bm = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                   fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  {  // max over the four j-lanes of the column (lanes l^16, l^32)
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
  }
  rescale_on_growth(st.m, bm, slack, c2, [&](float alpha) {
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      st.o[i] *= alpha;
      st.acc[i] *= alpha;
    }
    st.corr *= alpha;
    st.mt *= alpha;
  });
  const float nmc = -(st.m == -INFINITY ? 0.0f : st.m) * c2;
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c2, nmc));
  st.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// One K4V4 block in the grouped layout, in two phases.  Lane (column c, j);
// g = c & 3.
//  A: stage V codes and metadata through the wave's LDS area (metadata by
//     group: km[32 g + t], vm[32 g + t]), read back this lane's operands,
//     run the QK MFMAs and apply the K scales and mins -> raw scores.
//  B: online softmax, P' = s_v P, PV + bias + min-term MFMAs.
struct K4Mid {
  float s[8];                       // raw scores of the lane's tokens (head c >> 2)
  uint32_t vc[8];                   // V code dword c of the lane's eight tokens
  uint4 vma, vmb;                   // V {scale, min} of the tokens, group g
  uint4 mha, mhb;                   // V {scale, min} of the tokens, group c >> 2
};

// kVB = 2: 2-bit V codes, a 32-byte row per token (word w holds dims
// 16 w .. 16 w + 15).  Lane column c still owns output dims 8c .. 8c + 7:
// bits 16 (c & 1) .. + 15 of word c / 2, which phase B selects.
template <int kVB = 4, int kKB = 4>
__device__ __forceinline__ void k4_phase_a(K4Mid& x, const K4Raw& r, K4Stage& sg,
                                           const half8_t qg[4], float rc, float qsc,
                                           const Masks& k, int tb, int nq, int lane, int c, int j) {
  const int g = c & 3;
  wave_sync();
  if constexpr (kVB == 4) {
    *reinterpret_cast<uint4*>(&sg.v[lane >> 2][4 * (lane & 3)]) = r.va;
    *reinterpret_cast<uint4*>(&sg.v[16 + (lane >> 2)][4 * (lane & 3)]) = r.vb;
  } else {
    *reinterpret_cast<uint4*>(&sg.v[lane >> 1][4 * (lane & 1)]) = r.va;
  }
  {  // this lane loaded token lane/2, groups 2 (lane & 1) and 2 (lane & 1) + 1
    const int tm = lane >> 1, g0 = 2 * (lane & 1);
    sg.km[32 * g0 + tm] = r.kmw.x;
    sg.km[32 * (g0 + 1) + tm] = r.kmw.y;
    sg.vm[32 * g0 + tm] = r.vmw.x;
    sg.vm[32 * (g0 + 1) + tm] = r.vmw.y;
  }
  wave_sync();
  // {scale, min} of the lane's row tokens 4j + r (tile a) and 16 + 4j + r (tile b)
  const uint4 kma = *reinterpret_cast<const uint4*>(&sg.km[32 * g + 4 * j]);
  const uint4 kmb = *reinterpret_cast<const uint4*>(&sg.km[32 * g + 16 + 4 * j]);
  x.vma = *reinterpret_cast<const uint4*>(&sg.vm[32 * g + 4 * j]);
  x.vmb = *reinterpret_cast<const uint4*>(&sg.vm[32 * g + 16 + 4 * j]);
  // mins of the same tokens in group c >> 2: the A operand (row c) of the min term
  x.mha = *reinterpret_cast<const uint4*>(&sg.vm[32 * (c >> 2) + 4 * j]);
  x.mhb = *reinterpret_cast<const uint4*>(&sg.vm[32 * (c >> 2) + 16 + 4 * j]);
#pragma unroll
  for (int e = 0; e < 8; ++e) x.vc[e] = sg.v[k4_token(0, j, e)][kVB == 4 ? c : (c >> 1)];

  // accumulators start at -R, so they end at D - R
  float4_t da = {-rc, -rc, -rc, -rc}, db = {-rc, -rc, -rc, -rc};
  if constexpr (kKB == 4) {
    const uint32_t wa[4] = {r.ka.x, r.ka.y, r.ka.z, r.ka.w};
    const uint32_t wb[4] = {r.kb.x, r.kb.y, r.kb.z, r.kb.w};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      da = mfma(k_biased(wa[kk], k), qg[kk], da);
      db = mfma(k_biased(wb[kk], k), qg[kk], db);
    }
  } else {
    uint32_t m2, mg;
    asm volatile("v_mov_b32 %0, 0x03000300" : "=v"(m2));
    asm volatile("v_mov_b32 %0, 0x44004400" : "=v"(mg));
    // chunk kk: the low or high 16 bits of word kk / 2, bytes split into halves
    const uint32_t wa[2] = {r.ka.x, r.ka.y}, wb[2] = {r.kb.x, r.kb.y};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t sel = (kk & 1) ? 0x0C030C02u : 0x0C010C00u;
      da = mfma(k_biased2(__builtin_amdgcn_perm(0u, wa[kk >> 1], sel), m2, mg), qg[kk], da);
      db = mfma(k_biased2(__builtin_amdgcn_perm(0u, wb[kk >> 1], sel), m2, mg), qg[kk], db);
    }
  }
  const uint32_t ka4[4] = {kma.x, kma.y, kma.z, kma.w};
  const uint32_t kb4[4] = {kmb.x, kmb.y, kmb.z, kmb.w};
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const half2_t ma = as_half2(ka4[rr]), mb = as_half2(kb4[rr]);
    x.s[rr] = fmaf(static_cast<float>(ma[0]), da[rr], static_cast<float>(ma[1]) * qsc);
    x.s[4 + rr] = fmaf(static_cast<float>(mb[0]), db[rr], static_cast<float>(mb[1]) * qsc);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) x.s[e] = quad_sum(x.s[e]);
  if (tb + kBlk > nq) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (tb + 4 * j + e >= nq) x.s[e] = -INFINITY;
      if (tb + 16 + 4 * j + e >= nq) x.s[4 + e] = -INFINITY;
    }
  }
}

template <int kVB = 4>
__device__ __forceinline__ void k4_phase_b(GState& st, const K4Mid& x, const Masks& k, float c2, float slack,
                                           int c = 0) {
  float pr[8];
  softmax_g(st, x.s, c2, slack, pr);
  // B operands: P' = s_v P for the codes, P for the min term
  half8_t p16;
#pragma unroll
  for (int e = 0; e < 8; ++e) p16[e] = static_cast<_Float16>(pr[e]);
  // the V scales of the eight tokens, paired like the operand halves
  const half8_t sv = pack4(__builtin_amdgcn_perm(x.vma.y, x.vma.x, 0x05040100u),
                           __builtin_amdgcn_perm(x.vma.w, x.vma.z, 0x05040100u),
                           __builtin_amdgcn_perm(x.vmb.y, x.vmb.x, 0x05040100u),
                           __builtin_amdgcn_perm(x.vmb.w, x.vmb.z, 0x05040100u));
  const half8_t pp = p16 * sv;
  const half8_t am = pack4(__builtin_amdgcn_perm(x.mha.y, x.mha.x, 0x07060302u),
                           __builtin_amdgcn_perm(x.mha.w, x.mha.z, 0x07060302u),
                           __builtin_amdgcn_perm(x.mhb.y, x.mhb.x, 0x07060302u),
                           __builtin_amdgcn_perm(x.mhb.w, x.mhb.z, 0x07060302u));
  // V^T operands: biased codes, token pairs interleaved as in the generic path
  if constexpr (kVB == 4) {
    uint32_t xl[4], xh[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xl[q] = __builtin_amdgcn_perm(x.vc[2 * q + 1], x.vc[2 * q], 0x05040100u);
      xh[q] = __builtin_amdgcn_perm(x.vc[2 * q + 1], x.vc[2 * q], 0x07060302u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w = (i < 4) ? xl[q] : xh[q];
        if (i & 2) w >>= 8;
        v[q] = (w & ((i & 1) ? k.hi : k.lo)) | k.magic;
      }
      st.o[i] = mfma(pack4(v[0], v[1], v[2], v[3]), pp, st.o[i]);
    }
    st.corr = mfma(pack4(k.magic, k.magic, k.magic, k.magic), pp, st.corr);
  } else {
    // 2-bit codes: the lane's 16-bit half of each token's word (eight codes,
    // dim 8c + i at bits 2i), two tokens a register.  A code goes into
    // mantissa bits 8-9 under the exponent of 4 (0x4400 | c << 8 is exactly
    // 4 + c), so the bias is 4, not 1024: with codes of at most 3, a bias of
    // 1024 would leave the biased sums' fp32 rounding several hundred times
    // the size of the output's
    uint32_t m2, mg;
    asm volatile("v_mov_b32 %0, 0x03000300" : "=v"(m2));
    asm volatile("v_mov_b32 %0, 0x44004400" : "=v"(mg));
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = __builtin_amdgcn_perm(x.vc[2 * q + 1], x.vc[2 * q], sel);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = (i < 4) ? (xv[q] << (8 - 2 * i)) : (xv[q] >> (2 * i - 8));
        v[q] = (w & m2) | mg;
      }
      st.o[i] = mfma(pack4(v[0], v[1], v[2], v[3]), pp, st.o[i]);
    }
    st.corr = mfma(pack4(mg, mg, mg, mg), pp, st.corr);
  }
  st.mt = mfma(am, p16, st.mt);
}

// One FP16 block in the grouped layout: the same columns (no bias, no
// scale), P for even and 16 P for odd output dims, so that the FP16 and
// K4V4 contributions share one accumulator under O = (o - corr) (1 or 1/16) + mt
// (with kOdd16 off, P for every dim: the 2-bit V convention).
template <bool kOdd16 = true>
__device__ __forceinline__ void f16_compute_g(GState& st, const half8_t qf[4], const uint4 kr[8],
                                              const uint4 vr[8], int valid, int j, float c2, float slack) {
  float4_t da = {0.f, 0.f, 0.f, 0.f}, db = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    da = mfma(as_half8(kr[kk]), qf[kk], da);
    db = mfma(as_half8(kr[4 + kk]), qf[kk], db);
  }
  float s[8] = {da[0], da[1], da[2], da[3], db[0], db[1], db[2], db[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = quad_sum(s[e]);
  if (valid < kBlk) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * j + e >= valid) s[e] = -INFINITY;
      if (16 + 4 * j + e >= valid) s[4 + e] = -INFINITY;
    }
  }
  float pr[8];
  softmax_g(st, s, c2, slack, pr);
  half8_t p1, p16x;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p1[e] = static_cast<_Float16>(pr[e]);
    p16x[e] = p1[e] * static_cast<_Float16>(16.0f);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a0[4] = {vr[2 * q].x, vr[2 * q].y, vr[2 * q].z, vr[2 * q].w};
      const uint32_t a1[4] = {vr[2 * q + 1].x, vr[2 * q + 1].y, vr[2 * q + 1].z, vr[2 * q + 1].w};
      v[q] = __builtin_amdgcn_perm(a1[i >> 1], a0[i >> 1], sel);
    }
    st.o[i] = mfma(pack4(v[0], v[1], v[2], v[3]), (kOdd16 && (i & 1)) ? p16x : p1, st.o[i]);
  }
}




// ---------------------------------------------------------------------------
// Other code widths (K8V8, K4V2, K2V4, ...: b-bit keys and values, 8/b codes
// a byte).  A 32-token block of the quantised region is dequantised into a
// per-wave LDS tile of fp16 rows, then attended exactly like an FP16 block.
// Lane l owns half a row: token l / 2, elements 64 (l & 1) .. + 63 (two
// groups), whose codes and {scale, min} words it loads with wide loads.
// ---------------------------------------------------------------------------
constexpr int kTileStride = kD + 8;               // halves a row: 16-byte reads spread over banks
struct DqTile {
  uint16_t k[kBlk][kTileStride];
  uint16_t v[kBlk][kTileStride];
};

template <int kKB, int kVB>
struct GenRaw {
  uint4 k[kKB / 2];                 // 8 kKB code bytes of the lane's half row of K
  uint4 v[kVB / 2];
  uint2 km, vm;                     // {scale, min} of the half row's two groups
};

template <int kKB, int kVB>
__device__ __forceinline__ void load_gen(GenRaw<kKB, kVB>& r, const uint8_t* kq, const uint32_t* kmeta,
                                         const uint8_t* vq, const uint32_t* vmeta, int tb, int nq,
                                         int lane) {
  // rows past the unit's last token re-read it (masked below).  Ordinary
  // loads: each instruction takes 16 bytes a lane at a stride of 8 kKB
  // bytes, so the next instructions read the rest of the same lines, which
  // the non-temporal policy would not keep (K8V8 at B = 32: 669 us with it,
  // 452 us without)
  const uint32_t t = static_cast<uint32_t>(min(tb + (lane >> 1), nq - 1));
  const uint32_t h = lane & 1;
  const uint8_t* kp = kq + t * (16 * kKB) + h * (8 * kKB);
  const uint8_t* vp = vq + t * (16 * kVB) + h * (8 * kVB);
#pragma unroll
  for (int i = 0; i < kKB / 2; ++i) r.k[i] = ld16(kp + 16 * i);
#pragma unroll
  for (int i = 0; i < kVB / 2; ++i) r.v[i] = ld16(vp + 16 * i);
  r.km = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(kmeta) + t * 16 + h * 8);
  r.vm = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(vmeta) + t * 16 + h * 8);
}

// 64 b-bit codes (element e at bits b e .. of the little-endian words w) of
// two groups to 64 fp16 code * scale + min, each rounded once: a code goes
// under the exponent of 1024 (exactly 1024 + code, codes < 1024), 1024 is
// taken off, then one fused multiply-add.
template <int kB>
__device__ __forceinline__ void dq_half_row(uint16_t* dst, const uint32_t* w, uint2 meta) {
  constexpr uint32_t kMask = (1u << kB) - 1u;
  const half2_t k1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const half2_t sm = as_half2(g ? meta.y : meta.x);
    const half2_t s2 = {sm[0], sm[0]}, m2 = {sm[1], sm[1]};
    uint32_t o[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int e = 32 * g + 2 * p;
      const uint32_t c0 = (w[(kB * e) >> 5] >> ((kB * e) & 31)) & kMask;
      const uint32_t c1 = (w[(kB * (e + 1)) >> 5] >> ((kB * (e + 1)) & 31)) & kMask;
      const half2_t c = as_half2(c0 | (c1 << 16) | 0x64006400u) - k1024;
      o[p] = as_u32(__builtin_elementwise_fma(c, s2, m2));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      st16(dst + 32 * g + 8 * q, make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]));
  }
}

// The block's K and V as fp16 operands of the FP16-block code.
template <int kKB, int kVB>
__device__ __forceinline__ void gen_operands(uint4 kr[8], uint4 vr[8], const GenRaw<kKB, kVB>& r,
                                             DqTile& tl, int lane, int n, int j) {
  wave_sync();                                     // the previous block's reads are done
  const int t = lane >> 1, h = lane & 1;
  dq_half_row<kKB>(&tl.k[t][64 * h], reinterpret_cast<const uint32_t*>(r.k), r.km);
  dq_half_row<kVB>(&tl.v[t][64 * h], reinterpret_cast<const uint32_t*>(r.v), r.vm);
  wave_sync();
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kr[kk] = ld16(&tl.k[n][32 * j + 8 * kk]);
    kr[4 + kk] = ld16(&tl.k[16 + n][32 * j + 8 * kk]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) vr[e] = ld16(&tl.v[k4_token(0, j, e)][8 * n]);
}

// The blocks one wave of a unit scans: K4V4 blocks [k0, k1) (a contiguous
// range) and FP16 blocks f0, f0 + nwaves, ... below nblk_f.  An FP16 block
// moves wF = 512 / (bytes of a quantised token) times the bytes of a K4V4
// block (3.2 at K4V4), so the FP16 blocks go round-robin from wave 0 and the
// K4V4 blocks fill up to a common level: every wave gets about the same
// bytes whatever the mix.  Every wave evaluates the same float expressions
// for its own and its neighbour's boundary, so the ranges tile [0, nblk_q).
struct WaveWork {
  int k0, k1, f0;
};

__device__ __forceinline__ WaveWork wave_work(int gw, int nwaves, int nblk_q, int nblk_f, float wF) {
  const int full = nblk_f / nwaves, rem = nblk_f % nwaves;   // waves < rem hold full + 1 FP16 blocks
  const float cA = static_cast<float>(full + 1) * wF, cB = static_cast<float>(full) * wF;
  float level = (static_cast<float>(nblk_q) + rem * cA + (nwaves - rem) * cB) / nwaves;
  if (level < cA) level = cB + static_cast<float>(nblk_q) / (nwaves - rem);  // waves < rem take no K4V4 block
  const float kA = fmaxf(0.0f, level - cA), kB = fmaxf(0.0f, level - cB);
  auto start = [&](int w) {
    const float p = static_cast<float>(min(w, rem)) * kA + static_cast<float>(max(0, w - rem)) * kB;
    return min(nblk_q, static_cast<int>(p + 0.5f));
  };
  WaveWork r;
  r.k0 = start(gw);
  r.k1 = gw == nwaves - 1 ? nblk_q : start(gw + 1);
  r.f0 = gw;
  return r;
}

// LDS image of the waves' states for up to eight heads at a time:
// o[w][g][dim], plus each wave's running max and denominator per head.
constexpr int kImgHeads = 8;
struct WgImage {
  float o[kWaves][kImgHeads][kD];
  float m[kWaves][kImgHeads];
  float l[kWaves][kImgHeads];
};

// Per-thread partial of the final merge: (max, denominator, four dims).
struct FinPart {
  float m, l, pad0, pad1;
  float4_t o;
};

// Partial records cross XCDs.  They are written with device-scope (sc1)
// write-through stores and read with sc1 loads that miss the XCD-local L2,
// and the writer waits for its stores before counting its arrival, so no
// fence has to write back or invalidate a whole L2.
// 16-byte store with the device-scope write-through policy (sc1), so a
// record leaves in whole lines
__device__ __forceinline__ void st4_agent(float* p, float4_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}

template <bool kG4, int kKB, int kVB, bool kPaged>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  // K4V4 takes the grouped-code paths; other widths dequantise each block
  // into an LDS tile and use the FP16-block code
  constexpr bool kK4V4 = kKB == 4 && kVB == 4;
  // With G <= 4 the 2-bit widths (K4V2, K2V4, K2V2) take the grouped-code
  // path too: 2-bit codes are unpacked in registers as 4 + code (2-bit V:
  // every dim's operand, so the odd dims carry no 1/16 factor, kOdd16 off;
  // 2-bit K: no 1/16 query entries, R = 4 sum q)
  constexpr bool kGC = kG4 && (kKB == 2 || kKB == 4) && (kVB == 2 || kVB == 4);
  constexpr bool kK4G = kK4V4 || kGC;
  constexpr int kVC = kVB == 2 ? 2 : 4;
  constexpr int kKC = kKB == 2 ? 2 : 4;
  constexpr bool kOdd16 = !(kGC && kVB == 2);
  // bytes of an FP16 block over those of a quantised block (3.2 at K4V4)
  constexpr float kF16Weight = 512.0f / (16 * (kKB + kVB) + 32);
  using Stage = std::conditional_t<kK4G, K4Stage, DqTile>;
  // the per-wave staging areas of the scan, the image of the waves' states
  // and the partials of the final merge share LDS (barriers separate them)
  __shared__ union {
    Stage stage[kWaves];                           // 14 KB (K4 codes), 68 KB (tiles)
    WgImage img;                                   // 16.5 KB
    FinPart fin[kThreads];                         // 8 KB
  } s_lds;
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int n = lane & 15, j = lane >> 4;
  const int64_t u = blockIdx.y;
  const int split = blockIdx.x;
  const int nsplit = a.nsplit;
  const int G = a.G;
  const int64_t b = u / a.Hkv;
  const int h0 = static_cast<int>(u % a.Hkv) * G;
  const float c2 = a.c2;
  const float slack = a.slack;

  // Every lane ends its scan with one head's state: `valid` lanes hold
  // dims 32j + 8r + i (r < 4, i < 8) of head `head` in ofin[i][r]; m_h is the
  // head's running max and l_h the lane's share of its denominator.
  int head;
  bool valid;
  float m_h, l_h;
  float4_t ofin[8];
  if constexpr (kG4) {
    // lane (column c = n = 4h + g, j): the head and group of its column
    const int h = n >> 2, g = n & 3;
    const bool active = (g == j) && (h < G);
    // FP16 B operand: dims 32j + 8kk .. of head h where g == j, else zero
    half8_t qf[4], qg[4];
    {
      const uint16_t* qp = a.q + (b * a.Hq + h0 + min(h, G - 1)) * kD + 32 * j;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        qf[kk] = active ? as_half8(ld16(qp + 8 * kk)) : as_half8(make_uint4(0, 0, 0, 0));
        // K4V4 B operand: the unpack order {0,4,1,5,2,6,3,7}, high-nibble
        // entries (odd dims) scaled by 1/16
        const half8_t sh = __builtin_shufflevector(qf[kk], qf[kk], 0, 4, 1, 5, 2, 6, 3, 7);
        const _Float16 k16 = static_cast<_Float16>(kKC == 4 ? 0.0625f : 1.0f);
        qg[kk] = (half8_t){sh[0], sh[1], sh[2] * k16, sh[3] * k16, sh[4], sh[5], sh[6] * k16, sh[7] * k16};
      }
    }
    // R = bias * (sum of column c's operand entries: bias 1024, or 4 for
    // 2-bit keys) and qs = sum of group g
    // of head h (every j needs them, so each lane reads the group itself)
    float rc = 0.0f, qsc = 0.0f;
    if (h < G) {
      const uint16_t* qp = a.q + (b * a.Hq + h0 + h) * kD + 32 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8_t v = as_half8(ld16(qp + 8 * kk));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = static_cast<float>(v[e]);
          qsc += x;
          rc += (kKC == 4 && (e & 1)) ? static_cast<float>(v[e] * static_cast<_Float16>(0.0625f)) : x;
        }
      }
      rc *= kKC == 4 ? 1024.0f : 4.0f;
    }

    GState st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      st.o[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
      st.acc[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }
    st.corr = (float4_t){0.f, 0.f, 0.f, 0.f};
    st.mt = (float4_t){0.f, 0.f, 0.f, 0.f};

    const int nwaves = nsplit * kWaves;
    const int gw = split * kWaves + wave;
    const int nq = min(a.c.n_q[u], a.cap_q);
    const int nblk_q = (nq + kBlk - 1) / kBlk;
    const int nvl = min(a.c.n_vl[u], a.cap_vl);
    const int nst = a.k_new ? 1 : min(a.c.n_stg[u], a.cap_stg);
    const int nwin = unit_n_win(a, b);
    const int nf = nvl + nwin + nst;
    const int nblk_f = (nf + kBlk - 1) / kBlk;
    const WaveWork ww = wave_work(gw, nwaves, nblk_q, nblk_f, kF16Weight);
    const uint8_t* kq = a.c.kq + u * a.cap_q * (16 * kKB);
    const uint8_t* vq = a.c.vq + u * a.cap_q * (16 * kVB);
    const uint32_t* kmeta = reinterpret_cast<const uint32_t*>(a.c.kq_meta) + u * a.cap_q * kMetaWords;
    const uint32_t* vmeta = reinterpret_cast<const uint32_t*>(a.c.vq_meta) + u * a.cap_q * kMetaWords;
    // block bi of the unit's K4V4 slots: at the unit's base, or at its pool
    // block when the slots are paged (offsets then relative to the block,
    // the tail clamp inside it)
    auto blk_ptrs = [&](int bi, const uint8_t*& kb, const uint32_t*& kmb, const uint8_t*& vb,
                        const uint32_t*& vmb, int& tb, int& nqb) {
      if constexpr (kPaged) {
        const int64_t fs = k4_slot(a.c.k4_pages, a.cap_q, u, bi * kBlk);
        kb = a.c.kq + fs * (16 * kKB);
        vb = a.c.vq + fs * (16 * kVB);
        kmb = reinterpret_cast<const uint32_t*>(a.c.kq_meta) + fs * kMetaWords;
        vmb = reinterpret_cast<const uint32_t*>(a.c.vq_meta) + fs * kMetaWords;
        tb = 0;
        nqb = nq - bi * kBlk;
      } else {
        kb = kq;
        vb = vq;
        kmb = kmeta;
        vmb = vmeta;
        tb = bi * kBlk;
        nqb = nq;
      }
    };
    auto ld_k4 = [&](K4Raw& r, int bi) {
      const uint8_t *kb, *vb;
      const uint32_t *kmb, *vmb;
      int tb, nqb;
      blk_ptrs(bi, kb, kmb, vb, vmb, tb, nqb);
      load_k4<kVC, kKC>(r, kb, kmb, vb, vmb, tb, nqb, lane, n, j);
    };
    auto ld_gen = [&](GenRaw<kKB, kVB>& r, int bi) {
      const uint8_t *kb, *vb;
      const uint32_t *kmb, *vmb;
      int tb, nqb;
      blk_ptrs(bi, kb, kmb, vb, vmb, tb, nqb);
      load_gen(r, kb, kmb, vb, vmb, tb, nqb, lane);
    };
    F16Rows f;
    f.kvl = a.c.kvl + u * a.cap_vl * kD;
    f.vvl = a.c.vvl + u * a.cap_vl * kD;
    f.kwin = a.W > 0 ? a.c.kwin + u * a.W * kD : nullptr;
    f.vwin = a.W > 0 ? a.c.vwin + u * a.W * kD : nullptr;
    f.kstg = a.k_new ? a.k_new + u * kD : a.c.kstg + u * a.cap_stg * kD;
    f.vstg = a.k_new ? a.v_new + u * kD : a.c.vstg + u * a.cap_stg * kD;
    f.nvl = nvl;
    f.nwin = nwin;
    f.nf = nf;
    // A wave's FP16 blocks come first: the K and V rows of the first one
    // and the wave's first quantised block are in flight together before
    // any compute, so no load latency is left exposed between the two
    // parts.  Later FP16 blocks have their K rows loaded one block ahead.
    const bool has_f = ww.f0 < nblk_f, has_k = ww.k0 < ww.k1;
    uint4 kcur[8], vcur[8];
    if (has_f) {
      load_f16_k(kcur, f, ww.f0 * kBlk, n, j);
      load_f16_v(vcur, f, ww.f0 * kBlk, n, j);
    }
    // one block of prefetch in two alternating buffers (no register copies);
    // the loads are unconditional (past the end they re-read the wave's last
    // block) so that the wait before a compute only covers its own loads
    const int last = ww.k1 - 1;
    if constexpr (kK4G) {
      K4Stage& sg = s_lds.stage[wave];
      const Masks km = make_masks();
      K4Raw ra, rb;
      K4Mid x;
      if (has_k) ld_k4(ra, ww.k0);
      if (has_f) {
        int blk = ww.f0;
        for (; blk + nwaves < nblk_f; blk += nwaves) {
          uint4 knxt[8];
          load_f16_k(knxt, f, (blk + nwaves) * kBlk, n, j);
          f16_compute_g<kOdd16>(st, qf, kcur, vcur, nf - blk * kBlk, j, c2, slack);
#pragma unroll
          for (int e = 0; e < 8; ++e) kcur[e] = knxt[e];
          load_f16_v(vcur, f, (blk + nwaves) * kBlk, n, j);
        }
        f16_compute_g<kOdd16>(st, qf, kcur, vcur, nf - blk * kBlk, j, c2, slack);
      }
      if (has_k) {
        int blk = ww.k0;
        for (; blk < ww.k1; blk += 2) {
          ld_k4(rb, min(blk + 1, last));
          k4_phase_a<kVC, kKC>(x, ra, sg, qg, rc, qsc, km, blk * kBlk, nq, lane, n, j);
          k4_phase_b<kVC>(st, x, km, c2, slack, n);
          if (blk + 1 >= ww.k1) break;
          ld_k4(ra, min(blk + 2, last));
          k4_phase_a<kVC, kKC>(x, rb, sg, qg, rc, qsc, km, (blk + 1) * kBlk, nq, lane, n, j);
          k4_phase_b<kVC>(st, x, km, c2, slack, n);
          if ((blk + 2 - ww.k0) % kFlushBlocks == 0) flush_g<kOdd16>(st);
        }
      }
    } else {
      DqTile& tl = s_lds.stage[wave];
      GenRaw<kKB, kVB> ra, rb;
      if (has_k) ld_gen(ra, ww.k0);
      if (has_f) {
        int blk = ww.f0;
        for (; blk + nwaves < nblk_f; blk += nwaves) {
          uint4 knxt[8];
          load_f16_k(knxt, f, (blk + nwaves) * kBlk, n, j);
          f16_compute_g<kOdd16>(st, qf, kcur, vcur, nf - blk * kBlk, j, c2, slack);
#pragma unroll
          for (int e = 0; e < 8; ++e) kcur[e] = knxt[e];
          load_f16_v(vcur, f, (blk + nwaves) * kBlk, n, j);
        }
        f16_compute_g<kOdd16>(st, qf, kcur, vcur, nf - blk * kBlk, j, c2, slack);
      }
      if (has_k) {
        int blk = ww.k0;
        for (; blk < ww.k1; blk += 2) {
          uint4 kr[8], vr[8];
          ld_gen(rb, min(blk + 1, last));
          gen_operands(kr, vr, ra, tl, lane, n, j);
          f16_compute_g<kOdd16>(st, qf, kr, vr, nq - blk * kBlk, j, c2, slack);
          if (blk + 1 >= ww.k1) break;
          ld_gen(ra, min(blk + 2, last));
          gen_operands(kr, vr, rb, tl, lane, n, j);
          f16_compute_g<kOdd16>(st, qf, kr, vr, nq - (blk + 1) * kBlk, j, c2, slack);
        }
      }
    }
    // the head's state, unbiased: acc + (o - corr) (1 or 1/16) + mt
    head = h;
    valid = active;
    m_h = st.m;
    l_h = st.l;
    flush_g<kOdd16>(st);
#pragma unroll
    for (int i = 0; i < 8; ++i) ofin[i] = st.acc[i];
  } else {
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

    // The unit's work: its K4V4 blocks, then its FP16 blocks (vertical
    // lines, window, staging), 32 tokens each; wave w of workgroup `split` is
    // wave gw of the unit's nsplit * 4 and scans the blocks wave_work gives it.
    const int nwaves = nsplit * kWaves;
    const int gw = split * kWaves + wave;
    const int nq = min(a.c.n_q[u], a.cap_q);
    const int nblk_q = (nq + kBlk - 1) / kBlk;
    const int nvl = min(a.c.n_vl[u], a.cap_vl);
    const int nst = a.k_new ? 1 : min(a.c.n_stg[u], a.cap_stg);
    const int nwin = unit_n_win(a, b);
    const int nf = nvl + nwin + nst;
    const int nblk_f = (nf + kBlk - 1) / kBlk;
    const WaveWork ww = wave_work(gw, nwaves, nblk_q, nblk_f, kF16Weight);
    const uint8_t* kq = a.c.kq + u * a.cap_q * (16 * kKB);
    const uint8_t* vq = a.c.vq + u * a.cap_q * (16 * kVB);
    const uint32_t* kmeta = reinterpret_cast<const uint32_t*>(a.c.kq_meta) + u * a.cap_q * kMetaWords;
    const uint32_t* vmeta = reinterpret_cast<const uint32_t*>(a.c.vq_meta) + u * a.cap_q * kMetaWords;
    // block bi of the unit's K4V4 slots: at the unit's base, or at its pool
    // block when the slots are paged (offsets then relative to the block,
    // the tail clamp inside it)
    auto blk_ptrs = [&](int bi, const uint8_t*& kb, const uint32_t*& kmb, const uint8_t*& vb,
                        const uint32_t*& vmb, int& tb, int& nqb) {
      if constexpr (kPaged) {
        const int64_t fs = k4_slot(a.c.k4_pages, a.cap_q, u, bi * kBlk);
        kb = a.c.kq + fs * (16 * kKB);
        vb = a.c.vq + fs * (16 * kVB);
        kmb = reinterpret_cast<const uint32_t*>(a.c.kq_meta) + fs * kMetaWords;
        vmb = reinterpret_cast<const uint32_t*>(a.c.vq_meta) + fs * kMetaWords;
        tb = 0;
        nqb = nq - bi * kBlk;
      } else {
        kb = kq;
        vb = vq;
        kmb = kmeta;
        vmb = vmeta;
        tb = bi * kBlk;
        nqb = nq;
      }
    };
    auto ld_k4 = [&](K4Raw& r, int bi) {
      const uint8_t *kb, *vb;
      const uint32_t *kmb, *vmb;
      int tb, nqb;
      blk_ptrs(bi, kb, kmb, vb, vmb, tb, nqb);
      load_k4(r, kb, kmb, vb, vmb, tb, nqb, lane, n, j);
    };
    auto ld_gen = [&](GenRaw<kKB, kVB>& r, int bi) {
      const uint8_t *kb, *vb;
      const uint32_t *kmb, *vmb;
      int tb, nqb;
      blk_ptrs(bi, kb, kmb, vb, vmb, tb, nqb);
      load_gen(r, kb, kmb, vb, vmb, tb, nqb, lane);
    };
    F16Rows f;
    f.kvl = a.c.kvl + u * a.cap_vl * kD;
    f.vvl = a.c.vvl + u * a.cap_vl * kD;
    f.kwin = a.W > 0 ? a.c.kwin + u * a.W * kD : nullptr;
    f.vwin = a.W > 0 ? a.c.vwin + u * a.W * kD : nullptr;
    f.kstg = a.k_new ? a.k_new + u * kD : a.c.kstg + u * a.cap_stg * kD;
    f.vstg = a.k_new ? a.v_new + u * kD : a.c.vstg + u * a.cap_stg * kD;
    f.nvl = nvl;
    f.nwin = nwin;
    f.nf = nf;
    // A wave's FP16 blocks come first: the K and V rows of the first one
    // and the wave's first quantised block are in flight together before
    // any compute, so no load latency is left exposed between the two
    // parts.  Later FP16 blocks have their K rows loaded one block ahead.
    const bool has_f = ww.f0 < nblk_f, has_k = ww.k0 < ww.k1;
    uint4 kcur[8], vcur[8];
    if (has_f) {
      load_f16_k(kcur, f, ww.f0 * kBlk, n, j);
      load_f16_v(vcur, f, ww.f0 * kBlk, n, j);
    }
    const int last = ww.k1 - 1;
    half8_t qn[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qn[kk] = as_half8(qraw[kk]);
    auto f16_part = [&]() {
      if (!has_f) return;
      int blk = ww.f0;
      for (; blk + nwaves < nblk_f; blk += nwaves) {
        uint4 knxt[8];
        load_f16_k(knxt, f, (blk + nwaves) * kBlk, n, j);
        f16_compute(st, qn, kcur, vcur, nf - blk * kBlk, j, c2, slack);
#pragma unroll
        for (int e = 0; e < 8; ++e) kcur[e] = knxt[e];
        load_f16_v(vcur, f, (blk + nwaves) * kBlk, n, j);
      }
      f16_compute(st, qn, kcur, vcur, nf - blk * kBlk, j, c2, slack);
    };
    if constexpr (kK4V4) {
      half8_t qb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const half8_t nat = as_half8(qraw[kk]);
        qb[kk] = __builtin_shufflevector(nat, nat, 0, 4, 1, 5, 2, 6, 3, 7);
      }
      K4Stage& sg = s_lds.stage[wave];
      const Masks km = make_masks();
      K4Raw ra, rb;
      if (has_k) ld_k4(ra, ww.k0);
      f16_part();
      if (has_k) {
        int blk = ww.k0;
        for (; blk < ww.k1; blk += 2) {
          ld_k4(rb, min(blk + 1, last));
          compute_k4(st, ra, sg, qb, km, blk * kBlk, nq, lane, n, j, c2, slack);
          if (blk + 1 >= ww.k1) break;
          ld_k4(ra, min(blk + 2, last));
          compute_k4(st, rb, sg, qb, km, (blk + 1) * kBlk, nq, lane, n, j, c2, slack);
        }
      }
    } else {
      DqTile& tl = s_lds.stage[wave];
      GenRaw<kKB, kVB> ra, rb;
      if (has_k) ld_gen(ra, ww.k0);
      f16_part();
      if (has_k) {
        int blk = ww.k0;
        for (; blk < ww.k1; blk += 2) {
          uint4 kr[8], vr[8];
          ld_gen(rb, min(blk + 1, last));
          gen_operands(kr, vr, ra, tl, lane, n, j);
          f16_compute(st, qn, kr, vr, nq - blk * kBlk, j, c2, slack);
          if (blk + 1 >= ww.k1) break;
          ld_gen(ra, min(blk + 2, last));
          gen_operands(kr, vr, rb, tl, lane, n, j);
          f16_compute(st, qn, kr, vr, nq - (blk + 1) * kBlk, j, c2, slack);
        }
      }
    }
    head = n;
    valid = n < G;
    m_h = st.m;
    l_h = st.l;
#pragma unroll
    for (int i = 0; i < 8; ++i) ofin[i] = st.o[i];
  }

  // Merge the four waves' states and publish the workgroup's record.  The
  // waves write their states to LDS once; thread (head g, dims 4c..4c+3)
  // merges them and stores its part of the record with 16-byte device-scope
  // stores, at most eight heads per round.
  float* recs = a.part + u * nsplit * static_cast<int64_t>(G) * kPart;
  float lsum = l_h;                                // the head's denominator: sum over j
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  WgImage& img = s_lds.img;
  for (int g0 = 0; g0 < G; g0 += kImgHeads) {
    __syncthreads();                               // staging areas / previous round free
    const int gl = head - g0;
    if (gl >= 0 && gl < kImgHeads && valid) {
      float* o = &img.o[wave][gl][32 * j];         // dims 32j + 8r + i
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<float4_t*>(o + 8 * r) = (float4_t){ofin[0][r], ofin[1][r], ofin[2][r], ofin[3][r]};
        *reinterpret_cast<float4_t*>(o + 8 * r + 4) = (float4_t){ofin[4][r], ofin[5][r], ofin[6][r], ofin[7][r]};
      }
      if (j == 0) {
        img.m[wave][gl] = m_h;
        img.l[wave][gl] = lsum;
      }
    }
    __syncthreads();
    const int gn = min(kImgHeads, G - g0);
    if (tid < gn * (kD / 4)) {
      const int gl2 = tid >> 5, c = tid & 31;
      float mw[kWaves];
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = img.m[w][gl2];
        mx = fmaxf(mx, mw[w]);
      }
      float lt = 0.0f;
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
      if (mx != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = __builtin_amdgcn_exp2f((mw[w] - mx) * c2);
          lt = fmaf(f, img.l[w][gl2], lt);
          acc += f * *reinterpret_cast<const float4_t*>(&img.o[w][gl2][4 * c]);
        }
      }
      float* rec = recs + (static_cast<int64_t>(split) * G + g0 + gl2) * kPart;
      if (c == 0) st4_agent(rec, (float4_t){mx, lt, 0.0f, 0.0f});
      st4_agent(rec + 4 + 4 * c, acc);
    }
  }
  // every store of the record is complete before the arrival is counted
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(a.counters + u * kCounterStride, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == nsplit - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // the step's merge (its loads in flight during the fold), by the last wave
  // A decode step needs nothing staged (the new token takes the staging
  // slot's place in the scan); a unit that has a staged token is refused:
  // its outputs and LSE are NaN and its cache is left as it was.
  const bool refused = a.k_new && a.c.n_stg[u] != 0;
  const bool merger = a.k_new && !refused && wave == kWaves - 1;
  const int t_step = a.L_seq ? min(max(a.L_seq[b], 0), a.L_max) : a.L_max;
  StepIn step_in{};
  if (merger) step_in = step_load(a, u, t_step, lane);

  // the normalised output of (head g, dims 4c..4c+3) from its folded state
  auto finish = [&](int item, float mx, float lt, float4_t acc) {
    const int g = item >> 5, c = item & 31;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    uint16_t* dst = a.out + (b * a.Hq + h0 + g) * kD + 4 * c;
    uint2 pk;
    pk.x = (uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[0] * inv)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[1] * inv)) << 16);
    pk.y = (uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[2] * inv)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(acc[3] * inv)) << 16);
    if (refused) pk = make_uint2(0x7E007E00u, 0x7E007E00u);          // fp16 quiet NaNs
    *reinterpret_cast<uint2*>(dst) = pk;
    if (c == 0 && a.lse)
      a.lse[b * a.Hq + h0 + g] = refused ? __uint_as_float(0x7FC00000u)   // a quiet NaN
                                 : lt > 0.0f ? (mx * c2 + log2f(lt)) * 0.69314718055994531f : -INFINITY;
  };
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      recs, static_cast<short>(0), nsplit * G * kPart * 4, kRsrcWord3);

  // Every fold form below runs the same arithmetic on the same records in
  // the same order (fold16 for each partial, then combine_step over the S
  // partials in index order), so the outputs do not depend on the form: a
  // fused step's equal the plain decode's bit for bit.
  // fold16: partial pt takes 16 records (split indices s0, s0 + S, ...; past
  // nsplit masked) into its running state
  auto fold16 = [&](FinPart& pt, int s0, int S, const float2 (&ml)[16], const float4_t (&o4)[16]) {
    float m16[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) m16[k] = s0 + k * S < nsplit ? ml[k].x : -INFINITY;
    float mx = pt.m;
#pragma unroll
    for (int k = 0; k < 16; ++k) mx = fmaxf(mx, m16[k]);
    const float mu = mx == -INFINITY ? 0.0f : mx;
    const float fa = __builtin_amdgcn_exp2f((pt.m - mu) * c2);
    pt.l *= fa;
    pt.o *= fa;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float f = __builtin_amdgcn_exp2f((m16[k] - mu) * c2);
      pt.l = fmaf(f, ml[k].y, pt.l);
      pt.o += f * o4[k];
    }
    pt.m = mx;
  };
  auto load16 = [&](int s0, int S, int g, int c, float2 (&ml)[16], float4_t (&o4)[16]) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int sp = min(s0 + k * S, nsplit - 1);
      const int at = (sp * G + g) * kPart * 4;
      const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rs, at, 0, kSc1);
      ml[k] = make_float2(__uint_as_float(v2[0]), __uint_as_float(v2[1]));
      o4[k] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, at + 16 + 16 * c, 0, kSc1));
    }
  };
  // combine: partial w of the output (w < S), in order
  auto combine_step = [&](float& mx, float& lt, float4_t& acc, float m, float l, float4_t o) {
    const float f = __builtin_amdgcn_exp2f((m - mx) * c2);
    lt = fmaf(f, l, lt);
    acc += f * o;
  };

  // A fused step on the G <= 4 scan with two partials per output (G = 3, 4)
  // and at most 32 splits: the threads of the outputs (waves 0 and 1) each
  // load both partials' records in one round and fold and combine them in
  // registers, while the last wave, which has no output, runs the step's
  // merge beside them (after the fold it would add its quantisation and
  // stores to the step's tail).
  bool folded = false;
  if constexpr (kG4) {
    const int items = G * (kD / 4);
    if (a.k_new && kThreads / items == 2 && nsplit <= 32) {
      folded = true;
      if (merger) step_store<kKB, kVB>(a, u, t_step, lane, step_in);
      if (tid < items) {
        const int g = tid >> 5, c = tid & 31;
        float2 ml0[16], ml1[16];
        float4_t o40[16], o41[16];
        load16(0, 2, g, c, ml0, o40);
        load16(1, 2, g, c, ml1, o41);
        FinPart p0{-INFINITY, 0.0f, 0.0f, 0.0f, {0.f, 0.f, 0.f, 0.f}};
        FinPart p1 = p0;
        fold16(p0, 0, 2, ml0, o40);
        fold16(p1, 1, 2, ml1, o41);
        float mx = fmaxf(fmaxf(-INFINITY, p0.m), p1.m);
        float lt = 0.0f;
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (mx != -INFINITY) {
          combine_step(mx, lt, acc, p0.m, p0.l, p0.o);
          combine_step(mx, lt, acc, p1.m, p1.l, p1.o);
        }
        finish(tid, mx, lt, acc);
      }
    }
  }
  if (!folded) {
    // Otherwise the last workgroup merges the unit's nsplit * G records: thread (sub,
    // head g, dims 4c..4c+3) folds the records of its output with split index
    // sub, sub + S, ..., 16 at a time with all their loads in flight (device-
    // scope buffer loads: 8 bytes of (max, sum) and 16 of the output per
    // record).  The S partials of an output are then combined in LDS.  (Staging
    // whole records through LDS first, with fewer and wider loads, measured
    // slower: 17.5 against 16.8 us for the B = 1 launch.)
    const int items = G * (kD / 4);
    const int S = max(1, kThreads / items);
    const int sub = tid / items;
    const int n_items = (items + kThreads - 1) / kThreads;
    FinPart part[kFoldItems];
#pragma unroll
    for (int q = 0; q < kFoldItems; ++q) part[q] = FinPart{-INFINITY, 0.0f, 0.0f, 0.0f, {0.f, 0.f, 0.f, 0.f}};
    if (S == 2 && nsplit <= 32) {
      // G = 3, 4 with one batch per partial: lane l of wave w folds partial
      // l / 32 of output 32 w + l % 32, and the two partials of an output
      // meet across the wave's halves (a lane exchange, no LDS round and no
      // barrier), combined in the same order as below
      const int wl = tid & 63, it = (tid >> 6) * 32 + (wl & 31), sb = wl >> 5;
      const int ic = min(it, items - 1);
      FinPart pt{-INFINITY, 0.0f, 0.0f, 0.0f, {0.f, 0.f, 0.f, 0.f}};
      {
        float2 ml[16];
        float4_t o4[16];
        load16(sb, 2, ic >> 5, ic & 31, ml, o4);
        fold16(pt, sb, 2, ml, o4);
      }
      const float om = __shfl_xor(pt.m, 32), ol = __shfl_xor(pt.l, 32);
      const float4_t oo = {__shfl_xor(pt.o[0], 32), __shfl_xor(pt.o[1], 32), __shfl_xor(pt.o[2], 32),
                           __shfl_xor(pt.o[3], 32)};
      if (sb == 0 && it < items) {
        float mx = fmaxf(fmaxf(-INFINITY, pt.m), om);
        float lt = 0.0f;
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (mx != -INFINITY) {
          combine_step(mx, lt, acc, pt.m, pt.l, pt.o);
          combine_step(mx, lt, acc, om, ol, oo);
        }
        finish(it, mx, lt, acc);
      }
    } else {
      if (n_items == 2 && nsplit <= 16) {
        // G > 8 with one batch per output: both outputs' loads in one round
        // (the same folds as the loop below, in the same order)
        const int i1 = min(kThreads + tid, items - 1);
        float2 ml0[16], ml1[16];
        float4_t o40[16], o41[16];
        load16(0, 1, tid >> 5, tid & 31, ml0, o40);
        load16(0, 1, i1 >> 5, i1 & 31, ml1, o41);
        fold16(part[0], 0, 1, ml0, o40);
        fold16(part[1], 0, 1, ml1, o41);
      } else {
#pragma unroll
        for (int q = 0; q < kFoldItems; ++q) {
          if (q >= n_items) break;
          const int item = n_items > 1 ? q * kThreads + tid : tid % items;
          if (item >= items || sub >= S) continue;
          const int g = item >> 5, c = item & 31;
          for (int s0 = sub; s0 < nsplit; s0 += 16 * S) {
            float2 ml[16];
            float4_t o4[16];
            load16(s0, S, g, c, ml, o4);
            fold16(part[q], s0, S, ml, o4);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kFoldItems; ++q) {
        if (q >= n_items) break;                       // uniform: every thread has the same n_items
        const int item = n_items > 1 ? q * kThreads + tid : tid % items;
        const bool active = item < items && sub < S;
        __syncthreads();                               // the fold area / previous round's partials are free
        s_lds.fin[tid] = part[q];
        __syncthreads();
        if (active && sub == 0) {
          float mx = -INFINITY;
          for (int w = 0; w < S; ++w) mx = fmaxf(mx, s_lds.fin[tid + w * items].m);
          float lt = 0.0f;
          float4_t acc = {0.f, 0.f, 0.f, 0.f};
          if (mx != -INFINITY) {
            for (int w = 0; w < S; ++w) {
              const FinPart& pw = s_lds.fin[tid + w * items];
              combine_step(mx, lt, acc, pw.m, pw.l, pw.o);
            }
          }
          finish(item, mx, lt, acc);
        }
      }
    }
    if (merger) step_store<kKB, kVB>(a, u, t_step, lane, step_in);
  }
  if (tid == 0) a.counters[u * kCounterStride] = 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of hq_decode_attn_noalloc (for callers that cannot
// allocate): the arrival counters and partial records a decode workspace
// carries otherwise.  One copy per GPU, held until the process ends; every
// call on a GPU shares it.  In host code the array's name is only a stand-in:
// its device address comes from hipGetSymbolAddress, once per device, with
// that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero16_kernel(uint4* p, size_t n16) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t decode_scratch(void** ptr, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the arrival counters start at zero (a fill kernel, not a memset, so
    // that a captured first call records no memset node); every completed
    // call leaves the counters it used at zero again
    hipLaunchKernelGGL(zero16_kernel, dim3(64), dim3(256), 0, s, static_cast<uint4*>(p),
                       kScratchCounterBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const hq_dims& d, const hq_cache& c, int32_t L, const DecodePlan& plan,
                         const uint16_t* q, uint16_t* out, float* lse, void* ws, hipStream_t s,
                         const int32_t* L_seq, const uint16_t* k_new, const uint16_t* v_new,
                         const uint8_t* evict_is_vl) {
  return launch_decode_at(d, c, L, plan, q, out, lse, reinterpret_cast<int32_t*>(ws),
                          reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + decode_counter_bytes(d)),
                          s, L_seq, k_new, v_new, evict_is_vl);
}

hipError_t launch_decode_at(const hq_dims& d, const hq_cache& c, int32_t L, const DecodePlan& plan,
                            const uint16_t* q, uint16_t* out, float* lse, int32_t* counters,
                            float* part, hipStream_t s, const int32_t* L_seq,
                            const uint16_t* k_new, const uint16_t* v_new, const uint8_t* evict_is_vl) {
  DecodeArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.evict_is_vl = evict_is_vl;
  a.L_seq = L_seq;
  a.L_max = L;
  a.c = c;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.counters = counters;   // counter of unit u at word u * kCounterStride
  a.part = part;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.G = d.Hq / d.Hkv;
  a.W = d.W;
  a.cap_q = d.cap_q;
  a.cap_vl = d.cap_vl;
  a.cap_stg = d.cap_stg;
  a.n_win = plan.n_win;
  a.nsplit = plan.nsplit;
  a.c2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(d.d)));
  a.slack = 8.0f / a.c2;
  (void)L;
  dim3 grid(plan.nsplit, d.B * d.Hkv);
  const int kb = kv_bits(d.k_bits), vb = kv_bits(d.v_bits);
  // paged K4V4 slots are a template parameter: the contiguous instances
  // keep their block loads free of the page-table branch
  auto launch = [&](auto g4, auto kbc, auto vbc) {
    if (c.k4_pages)
      hipLaunchKernelGGL((decode_kernel<decltype(g4)::value, decltype(kbc)::value, decltype(vbc)::value, true>),
                         grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<decltype(g4)::value, decltype(kbc)::value, decltype(vbc)::value, false>),
                         grid, dim3(kThreads), 0, s, a);
  };
  auto by_v = [&](auto g4, auto kbc) {
    if (vb == 2) launch(g4, kbc, std::integral_constant<int, 2>{});
    else if (vb == 8) launch(g4, kbc, std::integral_constant<int, 8>{});
    else launch(g4, kbc, std::integral_constant<int, 4>{});
  };
  auto by_k = [&](auto g4) {
    if (kb == 2) by_v(g4, std::integral_constant<int, 2>{});
    else if (kb == 8) by_v(g4, std::integral_constant<int, 8>{});
    else by_v(g4, std::integral_constant<int, 4>{});
  };
  if (a.G <= 4) by_k(std::true_type{});
  else by_k(std::false_type{});
  return hipGetLastError();
}

}  // namespace hq
